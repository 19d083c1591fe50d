/*
 * msim_host.cpp -- host side of the C ABI declared in include/msim.h.
 *
 * msim_create validates the batch and compiles every experiment into one
 * arena (see msim_layout.h): ports numbered by cable order, up/down shortest
 * path routes with ECMP (Multiverse section 5: ECMP load balancing; the
 * candidate order and hash are this library's reading), the collectives'
 * point-to-point connections and flow schedules (Multiverse section 3.1: the
 * system simulator produces point-to-point flows from NCCL's collective
 * algorithms; AutoCCL section 2.3: NC channels moving chunks of size C one
 * after the other; AlpaComm section 3.1 Fig. 3d: pipelined broadcast), and the
 * initial mutable state.  msim_bind uploads the arenas; msim_run launches the
 * megakernel; msim_results reads the per-experiment totals back.
 */
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <string>
#include <thread>
#include <vector>

#include "msim.h"
#include "msim_layout.h"

static_assert(CC_DCTCP == MSIM_CC_DCTCP && CC_DCQCN == MSIM_CC_DCQCN && CC_HPCC == MSIM_CC_HPCC, "congestion-control codes");

extern "C" hipError_t msim_launch_run(const KParams *kp, uint32_t kind, uint32_t grid, uint32_t block,
                                      uint32_t lds, uint32_t *clear, uint32_t n_clear, hipStream_t stream);
extern "C" hipError_t msim_scratch_words(uint32_t **out);
extern "C" hipError_t msim_launch_reset(const KParams *kp, uint64_t o_rec_all, uint64_t rec_words,
                                        hipStream_t stream);
extern "C" hipError_t msim_occupancy(uint32_t kind, uint32_t block, uint32_t lds, int *blocks_per_cu);
extern "C" hipError_t msim_set_lds_limit(uint32_t kind, uint32_t lds);

namespace {

thread_local std::string g_create_error;

/* LDS a compact arena may use (gfx950: 160 KiB per workgroup, less the
 * kernel's static reductions area) */
constexpr uint32_t COMPACT_LDS_LIMIT = 160u * 1024u - 4096u;

struct Compiled {
    std::vector<uint8_t> arena;  /* RO + initial RW image, size multiple of 16 */
    uint32_t rw_off = 0, bytes = 0, lds_bytes = 0;
    bool compact = false;
    uint32_t kind = 0;     /* kernel kind: 0 general; compact 1 + (16-byte rows << 2 | 32-bit descriptors << 1 | rate > 1);
                              KIND_GENERAL_TASKS: general with a task graph;
                              KIND_GENERAL_CC: general with congestion control */
    uint32_t nt = 0;       /* compact: thread slots */
    uint64_t n_flows = 0, n_conns = 0, n_ports = 0;
    uint64_t est_hops = 0, est_delivered = 0;
    uint64_t est_ticks = 0;  /* busiest link: packets over rate, flows on their ECMP paths (a lower bound on ticks unless sprayed) */
    uint64_t ring_pmin = 0;  /* smallest ring chunk in packets (0: no ring) */
    uint32_t n_task = 0, o_trw = 0;   /* task graph (general format) */
    uint32_t split_bytes = 0;         /* general format: LDS bytes of the switch/NIC state alone */
    uint32_t port_bytes = 0;          /* general format: LDS bytes of the port table alone */
    int err = 0;
    std::string msg;
};

uint32_t fmix32(uint32_t h)
{
    /* MurmurHash3 32-bit finaliser (Appleby, public domain) */
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

int fail(Compiled &c, int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c.err = code;
    c.msg = buf;
    return code;
}

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

/* One connection before layout. */
struct Conn {
    uint32_t src, dst, grp, idx;
    uint32_t route = 0, links = 0, lidx = 0, lat = 0;
    uint64_t pkts = 0;
};

/* Chunk rank i sends at step s of a ring round. */
uint32_t ring_chunk(uint32_t kind, uint32_t N, uint32_t i, uint32_t s)
{
    if (kind == GK_RING_AG || s < N - 1) return (i + N - s) % N;
    uint32_t s2 = s - (N - 1);
    return (i + 1 + N - s2) % N;
}

/* Flows each connection of group g carries, in sending order. */
uint32_t flows_per_conn(const Grp &g)
{
    switch (g.kind) {
    case GK_BCAST: return g.S;
    case GK_XFLOW:
    case GK_SEQ: return 1u;
    case GK_TREE: return g.R;
    default: return g.R * g.S;
    }
}

/* Connections of group g. */
uint32_t conns_of(const Grp &g)
{
    return g.kind == GK_TREE ? 2 * (g.N - 1) : g.N;
}

uint32_t first_flow_size(const Grp &g, uint32_t idx)
{
    if (g.kind == GK_XFLOW) return idx;
    if (g.kind == GK_SEQ) return g.p;
    if (g.kind == GK_TREE) return g.R > 1 ? g.p : g.X;
    if (g.kind == GK_BCAST) return g.p / g.S + (0 < g.p % g.S ? 1u : 0u);
    if (g.R > 1) return g.p;
    uint32_t k = ring_chunk(g.kind, g.N, idx, 0);
    return g.X / g.N + (k < g.X % g.N ? 1u : 0u);
}

/* Whether the groups fit the ring format: ring channels without gates, few
 * enough to index in a descriptor, each with flows that fit its fields. */
bool ngrp_fits_ring(const std::vector<Grp> &grp)
{
    if (grp.empty() || grp.size() > RING_MAX_GRP) return false;
    for (const Grp &g : grp) {
        if (g.kind != GK_RING_AR && g.kind != GK_RING_AG) return false;
        if (g.link != MSIM_NONE || g.N > RING_MAX_N || (uint64_t)g.R * g.S > C_POS_MASK) return false;
        if (g.p >= 65535u || g.X / g.N + 1 >= 65535u) return false;
    }
    return true;
}

/* Staging words of the ring format.  Port slot u's word is read by u and
 * written by the port at the far end of u's cable; stg[u] is chosen so that
 * the 64 lanes of every wavefront read 64 different LDS banks and write 64
 * different banks.  It is a proper colouring, with 64 colours, of the edges
 * u: (u's wavefront as reader, its far end's wavefront as writer) of a
 * bipartite multigraph in which no node has more than 64 edges, so such a
 * colouring exists (Konig); it is built edge by edge: take a colour ca free
 * at the reader and cb free at the writer; if ca is taken at the writer, swap
 * ca and cb along the path of ca / cb edges that starts there (the path
 * cannot reach the reader, which has no ca edge), which frees ca at the
 * writer.  The slots of colour c take c, c + 64, c + 128, ...  Returns false
 * if a check of the result fails. */
bool ring_staging(const std::vector<uint32_t> &slot, const std::vector<PortRO> &port, uint32_t n_ports, uint32_t nt,
                  std::vector<uint32_t> &stg)
{
    const uint32_t NW = (nt + 63) / 64;
    std::vector<int32_t> at_r((size_t)NW * 64, -1), at_w((size_t)NW * 64, -1), col(n_ports, -1);
    std::vector<uint32_t> rw(n_ports), ww(n_ports);
    for (uint32_t q = 0; q < n_ports; q++) {
        rw[q] = slot[q] / 64;
        ww[q] = slot[port[q].peer] / 64;
    }
    std::vector<int32_t> path;
    for (uint32_t q = 0; q < n_ports; q++) {
        const uint32_t a = rw[q], b = ww[q];
        int32_t ca = -1, cb = -1;
        for (int32_t c = 0; c < 64 && ca < 0; c++)
            if (at_r[a * 64 + c] < 0) ca = c;
        for (int32_t c = 0; c < 64 && cb < 0; c++)
            if (at_w[b * 64 + c] < 0) cb = c;
        if (ca < 0 || cb < 0) return false;
        if (at_w[b * 64 + ca] >= 0) {
            path.clear();
            uint32_t node = b;
            bool writer = true;
            int32_t c = ca;
            for (;;) {
                const int32_t e = writer ? at_w[node * 64 + c] : at_r[node * 64 + c];
                if (e < 0) break;
                path.push_back(e);
                node = writer ? rw[e] : ww[e];
                writer = !writer;
                c = c == ca ? cb : ca;
            }
            for (int32_t e : path) {
                at_r[rw[e] * 64 + col[e]] = -1;
                at_w[ww[e] * 64 + col[e]] = -1;
            }
            for (int32_t e : path) {
                col[e] = col[e] == ca ? cb : ca;
                at_r[rw[e] * 64 + col[e]] = e;
                at_w[ww[e] * 64 + col[e]] = e;
            }
        }
        col[q] = ca;
        at_r[a * 64 + ca] = (int32_t)q;
        at_w[b * 64 + ca] = (int32_t)q;
    }
    stg.assign(nt, 0);
    std::vector<uint32_t> cnt(64, 0);
    for (uint32_t q = 0; q < n_ports; q++) stg[slot[q]] = (uint32_t)col[q] + 64u * cnt[col[q]]++;
    /* checks: every word below NW * 64 and used once; within a wavefront, the
     * words read and the words written fall in 64 different banks */
    std::vector<uint8_t> used((size_t)NW * 64, 0);
    std::vector<uint64_t> rb(NW, 0), wb(NW, 0);
    for (uint32_t q = 0; q < n_ports; q++) {
        const uint32_t w = stg[slot[q]];
        if (w >= NW * 64 || used[w]) return false;
        used[w] = 1;
        const uint64_t bit = 1ull << (w & 63);
        const uint32_t wr = slot[port[q].peer] / 64;     /* the wavefront writing this word */
        if ((rb[rw[q]] & bit) || (wb[wr] & bit)) return false;
        rb[rw[q]] |= bit;
        wb[wr] |= bit;
    }
    return true;
}

/* Launch bound of each kernel kind (threads per workgroup). */
uint32_t kind_max_threads(uint32_t kind)
{
    if (kind == KIND_GENERAL_TASKS || kind == KIND_GENERAL_CC || kind == KIND_GENERAL_SPRAY) return 512u;
    if (kind == KIND_COMPACT_X8 || kind == KIND_COMPACT_X16) return COMPACT_X_THREADS;
    return 1024u;
}

int compile_exp(const msim_batch_spec *s, uint32_t e, bool allow_compact, bool allow_ring, Compiled &out)
{
    const uint32_t t = s->exp_topo[e], w = s->exp_work[e];
    if (t >= s->n_topo || w >= s->n_work) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: topology/workload index out of range", e);
    const uint32_t Q = s->exp_queue_pkts[e], seed = s->exp_ecmp_seed[e];
    const uint64_t pkt = s->exp_pkt_bytes[e];
    if (Q < 1 || Q > MSIM_MAX_QUEUE) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: queue %u outside 1..%u", e, Q, MSIM_MAX_QUEUE);
    if (pkt == 0) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: zero packet size", e);
    const uint32_t cc = s->exp_cc ? s->exp_cc[e] : MSIM_CC_NONE;
    uint32_t ecn_k = 0, cwnd0 = 0;
    if (cc > MSIM_CC_HPCC) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: unknown congestion control %u", e, cc);
    if (cc == MSIM_CC_DCTCP) {
        if (!s->exp_ecn_k || !s->exp_cwnd0) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: DCTCP needs exp_ecn_k and exp_cwnd0", e);
        ecn_k = s->exp_ecn_k[e];
        cwnd0 = s->exp_cwnd0[e];
        if (cwnd0 < 1 || cwnd0 > MSIM_MAX_CWND) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: initial window %u outside 1..%u", e, cwnd0, MSIM_MAX_CWND);
    }
    if (cc == MSIM_CC_DCQCN) {
        if (!s->exp_ecn_k) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: DCQCN needs exp_ecn_k", e);
        ecn_k = s->exp_ecn_k[e];
    }
    if (cc == MSIM_CC_HPCC) ecn_k = 0xFFFFFFFFu;     /* telemetry, no ECN marks */
    const uint32_t lb = s->exp_lb ? s->exp_lb[e] : MSIM_LB_ECMP;
    if (lb > MSIM_LB_SPRAY) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: unknown load balancing %u", e, lb);
    if (lb == MSIM_LB_SPRAY && cc != MSIM_CC_NONE)
        return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: packet spraying with congestion control is not supported", e);

    /* ---- topology: nodes, ports numbered by cable order */
    const uint32_t n0 = s->topo_node_off[t], nn = s->topo_node_off[t + 1] - n0;
    const uint32_t c0 = s->topo_cable_off[t], nc = s->topo_cable_off[t + 1] - c0;
    const uint8_t *layer = s->node_layer + n0;
    std::vector<uint32_t> deg(nn, 0);
    uint32_t maxd = 1, maxr = 1;
    for (uint32_t k = 0; k < nc; k++) {
        uint32_t a = s->cable_a[c0 + k], b = s->cable_b[c0 + k];
        if (a >= nn || b >= nn || a == b) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: cable %u has bad endpoints", e, k);
        if (layer[a] == layer[b]) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: cable %u joins two nodes of layer %u", e, k, layer[a]);
        uint32_t ra = s->cable_rate_ab[c0 + k], rb = s->cable_rate_ba[c0 + k], d = s->cable_delay[c0 + k];
        if (ra < 1 || rb < 1 || ra > MSIM_MAX_RATE || rb > MSIM_MAX_RATE) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: cable %u rate outside 1..%u", e, k, MSIM_MAX_RATE);
        if (d < 1 || d > MSIM_MAX_DELAY) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: cable %u delay outside 1..%u", e, k, MSIM_MAX_DELAY);
        maxd = std::max(maxd, d);
        maxr = std::max(maxr, std::max(ra, rb));
        deg[a]++;
        deg[b]++;
    }
    std::vector<uint32_t> pbase(nn + 1, 0), vbase(nn, 0), host_of(nn, MSIM_NONE);
    uint32_t n_voq = 0, n_hosts = 0;
    for (uint32_t n = 0; n < nn; n++) {
        if (layer[n] == 0) {
            if (deg[n] != 1) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: host node %u has %u cables (needs exactly 1)", e, n, deg[n]);
            host_of[n] = n_hosts++;
        } else {
            if (deg[n] > MSIM_MAX_SWITCH_PORTS) return fail(out, MSIM_E_LIMIT, "experiment %u: switch %u has %u ports (max %u)", e, n, deg[n], MSIM_MAX_SWITCH_PORTS);
            vbase[n] = n_voq;
            n_voq += deg[n] * deg[n];
        }
        pbase[n + 1] = pbase[n] + deg[n];
    }
    const uint32_t n_ports = pbase[nn];
    std::vector<PortRO> port(n_ports);
    std::vector<uint32_t> port_node(n_ports), fill(nn, 0);
    for (uint32_t k = 0; k < nc; k++) {
        uint32_t a = s->cable_a[c0 + k], b = s->cable_b[c0 + k];
        uint32_t pa = pbase[a] + fill[a]++, pb = pbase[b] + fill[b]++;
        bool alive = s->cable_alive[c0 + k] != 0;
        PortRO &A = port[pa], &B = port[pb];
        A.peer = pb; B.peer = pa;
        A.rate = s->cable_rate_ab[c0 + k]; B.rate = s->cable_rate_ba[c0 + k];
        A.delay = B.delay = s->cable_delay[c0 + k];
        A.alive = B.alive = alive ? 1 : 0;
        port_node[pa] = a; port_node[pb] = b;
    }
    for (uint32_t n = 0; n < nn; n++)
        for (uint32_t p = pbase[n]; p < pbase[n + 1]; p++) {
            PortRO &P = port[p];
            P.base = pbase[n];
            P.vbase = vbase[n];
            P.host = host_of[n];
            P.local = (uint8_t)(p - pbase[n]);
            P.deg = (uint8_t)deg[n];
            P.is_host = layer[n] == 0;
            P.peer_is_host = layer[port_node[P.peer]] == 0;
            P.pad = 0;
        }

    /* ---- workload: groups and connections */
    std::vector<Grp> grp;
    std::vector<Conn> conn;
    uint64_t fid = 0;
    auto is_host = [&](uint32_t h) { return h < nn && layer[h] == 0; };
    const uint32_t cw0 = s->work_coll_off[w];
    std::vector<uint32_t> grp_of_coll(s->work_coll_off[w + 1] - cw0, MSIM_NONE);   /* first group of each collective */
    for (uint32_t ci = s->work_coll_off[w]; ci < s->work_coll_off[w + 1]; ci++) {
        grp_of_coll[ci - cw0] = (uint32_t)grp.size();
        const uint32_t *mem = s->member_host + s->coll_member_off[ci];
        const uint32_t N = s->coll_member_off[ci + 1] - s->coll_member_off[ci];
        if (N < 2) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u has %u members", e, ci, N);
        for (uint32_t i = 0; i < N; i++) {
            if (!is_host(mem[i])) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u member %u is not a host", e, ci, mem[i]);
            for (uint32_t j = 0; j < i; j++)
                if (mem[j] == mem[i]) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u repeats host %u", e, ci, mem[i]);
        }
        const uint64_t P = (s->coll_bytes[ci] + pkt - 1) / pkt;
        const uint32_t type = s->coll_type[ci];
        const bool is_ring = type == MSIM_COLL_RING_ALLREDUCE || type == MSIM_COLL_RING_ALLGATHER ||
                             type == MSIM_COLL_RING_REDUCESCATTER;
        /* a ring may be gated on an earlier send/recv whose receivers are its members, in order */
        uint32_t gate_grp = MSIM_NONE;
        const uint32_t gate = s->coll_gate ? s->coll_gate[ci] : MSIM_NO_GATE;
        if (gate != MSIM_NO_GATE) {
            const uint32_t gi = cw0 + gate;
            if (!is_ring || gi >= ci || s->coll_type[gi] != MSIM_COLL_SENDRECV ||
                s->coll_member_off[gi + 1] - s->coll_member_off[gi] != N + 1)
                return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u has an invalid gate %u", e, ci, gate);
            for (uint32_t i = 0; i < N; i++)
                if (s->member_host[s->coll_member_off[gi] + 1 + i] != mem[i])
                    return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u: gate receivers differ from its members", e, ci);
            gate_grp = grp_of_coll[gate];
            if (grp[gate_grp].X != 0)
                return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: send/recv %u gates more than one collective", e, gi);
        }
        if (is_ring) {
            const uint32_t NC = s->coll_nc[ci];
            const uint64_t cb = s->coll_chunk_bytes[ci];
            if (NC < 1 || cb == 0 || cb % pkt) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u needs NC >= 1 and a chunk of whole packets", e, ci);
            const uint64_t p = cb / pkt;
            const uint32_t kind = type == MSIM_COLL_RING_ALLREDUCE ? GK_RING_AR : GK_RING_AG;   /* RS: as AG */
            if (gate_grp != MSIM_NONE) { grp[gate_grp].link = (uint32_t)grp.size(); grp[gate_grp].X = NC; }
            const uint32_t S = kind == GK_RING_AR ? 2 * (N - 1) : N - 1;
            for (uint32_t c = 0; c < NC; c++) {
                const uint64_t Pc = P / NC + (c < P % NC ? 1 : 0);
                if (Pc < N) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u channel %u carries %llu packets for %u ranks", e, ci, c, (unsigned long long)Pc, N);
                uint64_t R = (Pc + N * p - 1) / (N * p);
                uint64_t X = Pc - (R - 1) * N * p;
                if (R > 1 && X < N) { R--; X = Pc - (R - 1) * N * p; }
                if (R * S > CS_POS_MASK || p > 0xFFFFFFFFull || X > 0xFFFFFFFFull) return fail(out, MSIM_E_LIMIT, "experiment %u: collective %u too large", e, ci);
                Grp g{};
                g.kind = kind; g.N = N; g.S = S; g.R = (uint32_t)R; g.p = (uint32_t)p; g.X = (uint32_t)X;
                g.fid_base = (uint32_t)fid; g.conn_base = (uint32_t)conn.size(); g.link = gate_grp;
                out.ring_pmin = out.ring_pmin ? std::min<uint64_t>(out.ring_pmin, p) : p;
                fid += R * S * N;
                if (fid >= MSIM_NONE) return fail(out, MSIM_E_LIMIT, "experiment %u: too many flows", e);
                for (uint32_t i = 0; i < N; i++) {
                    Conn cn;
                    cn.src = mem[i]; cn.dst = mem[(i + 1) % N]; cn.grp = (uint32_t)grp.size(); cn.idx = i;
                    uint64_t last = 0;
                    for (uint32_t st = 0; st < S; st++) {
                        uint32_t k = ring_chunk(kind, N, i, st);
                        last += X / N + (k < X % N ? 1 : 0);
                    }
                    cn.pkts = (R - 1) * S * p + last;
                    conn.push_back(cn);
                }
                grp.push_back(g);
            }
        } else if (type == MSIM_COLL_PIPE_BROADCAST) {
            const uint64_t K = s->coll_k[ci];
            if (K < 1 || K > P || P > 0xFFFFFFFFull) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: broadcast %u needs 1 <= K <= packets", e, ci);
            const uint32_t A = N - 1;
            Grp g{};
            g.kind = GK_BCAST; g.N = A; g.S = (uint32_t)K; g.R = 1; g.p = (uint32_t)P; g.X = 0;
            g.fid_base = (uint32_t)fid; g.conn_base = (uint32_t)conn.size(); g.link = MSIM_NONE;
            fid += (uint64_t)A * K;
            if (fid >= MSIM_NONE) return fail(out, MSIM_E_LIMIT, "experiment %u: too many flows", e);
            for (uint32_t j = 1; j <= A; j++) {
                Conn cn;
                cn.src = mem[j - 1]; cn.dst = mem[j]; cn.grp = (uint32_t)grp.size(); cn.idx = j - 1; cn.pkts = P;
                conn.push_back(cn);
            }
            grp.push_back(g);
        } else if (type == MSIM_COLL_TREE_ALLREDUCE) {
            /* binary tree in member order; per channel: up connections of members
             * 1..N-1 (to their parent (i-1)/2), then down connections of 1..N-1 */
            const uint32_t NC = s->coll_nc[ci];
            const uint64_t cb = s->coll_chunk_bytes[ci];
            if (NC < 1 || cb == 0 || cb % pkt) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: tree %u needs NC >= 1 and a chunk of whole packets", e, ci);
            const uint64_t p = cb / pkt;
            for (uint32_t c = 0; c < NC; c++) {
                const uint64_t Pc = P / NC + (c < P % NC ? 1 : 0);
                if (Pc < 1) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: tree %u channel %u carries no packet", e, ci, c);
                const uint64_t R = (Pc + p - 1) / p;
                if (R > CS_POS_MASK || p > 0xFFFFFFFFull) return fail(out, MSIM_E_LIMIT, "experiment %u: tree %u too large", e, ci);
                Grp g{};
                g.kind = GK_TREE; g.N = N; g.S = 1; g.R = (uint32_t)R; g.p = (uint32_t)p;
                g.X = (uint32_t)(Pc - (R - 1) * p);
                g.fid_base = (uint32_t)fid; g.conn_base = (uint32_t)conn.size(); g.link = MSIM_NONE;
                fid += R * 2 * (N - 1);
                if (fid >= MSIM_NONE) return fail(out, MSIM_E_LIMIT, "experiment %u: too many flows", e);
                for (uint32_t j = 0; j < 2 * (N - 1); j++) {
                    const uint32_t i = j < N - 1 ? j + 1 : j - (N - 1) + 1;
                    Conn cn;
                    cn.src = j < N - 1 ? mem[i] : mem[(i - 1) / 2];
                    cn.dst = j < N - 1 ? mem[(i - 1) / 2] : mem[i];
                    cn.grp = (uint32_t)grp.size(); cn.idx = j; cn.pkts = Pc;
                    conn.push_back(cn);
                }
                grp.push_back(g);
            }
        } else if (type == MSIM_COLL_SENDRECV) {
            if (P < 1 || P > 0xFFFFFFFFull) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: send/recv %u needs 1 .. 2^32-1 packets", e, ci);
            Grp g{};
            g.kind = GK_SEQ; g.N = N - 1; g.S = 1; g.R = 1; g.p = (uint32_t)P; g.X = 0;
            g.fid_base = (uint32_t)fid; g.conn_base = (uint32_t)conn.size(); g.link = MSIM_NONE;
            fid += N - 1;
            if (fid >= MSIM_NONE) return fail(out, MSIM_E_LIMIT, "experiment %u: too many flows", e);
            for (uint32_t j = 1; j < N; j++) {
                Conn cn;
                cn.src = mem[0]; cn.dst = mem[j]; cn.grp = (uint32_t)grp.size(); cn.idx = j - 1; cn.pkts = P;
                conn.push_back(cn);
            }
            grp.push_back(g);
        } else {
            return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: collective %u has unknown type %u", e, ci, type);
        }
    }
    const uint32_t coll_grp_end = (uint32_t)grp.size();
    const uint64_t x0 = s->work_xflow_off[w], x1 = s->work_xflow_off[w + 1];
    if (x1 > x0) {
        Grp g{};
        g.kind = GK_XFLOW; g.N = (uint32_t)(x1 - x0); g.S = 1; g.R = 1;
        g.fid_base = (uint32_t)fid; g.conn_base = (uint32_t)conn.size(); g.link = MSIM_NONE;
        fid += x1 - x0;
        if (fid >= MSIM_NONE) return fail(out, MSIM_E_LIMIT, "experiment %u: too many flows", e);
        for (uint64_t xi = x0; xi < x1; xi++) {
            uint32_t a = s->xflow_src[xi], b = s->xflow_dst[xi], n = s->xflow_pkts[xi];
            if (!is_host(a) || !is_host(b) || a == b || n == 0) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: explicit flow %llu invalid", e, (unsigned long long)(xi - x0));
            Conn cn;
            cn.src = a; cn.dst = b; cn.grp = (uint32_t)grp.size(); cn.idx = n; cn.pkts = n;
            conn.push_back(cn);
        }
        grp.push_back(g);
    }
    if (conn.size() >= (1u << (31 - DESC_SHIFT))) return fail(out, MSIM_E_LIMIT, "experiment %u: too many connections", e);

    /* ---- task graph: validated as the spec states; a collective task's
     * groups carry the task's index */
    for (Grp &g : grp) g.task = MSIM_NONE;
    std::vector<TaskRO> tasks;
    std::vector<TaskRW> task_rw;
    std::vector<uint32_t> tpred;
    if (s->work_task_off) {
        const uint32_t t0 = s->work_task_off[w], t1 = s->work_task_off[w + 1];
        const uint32_t ncoll = s->work_coll_off[w + 1] - cw0;
        std::vector<uint8_t> named(ncoll, 0);
        for (uint32_t k = t0; k < t1; k++) {
            TaskRO tk{};
            TaskRW tw{};
            tw.start = tw.finish = MSIM_NONE;
            tk.type = s->task_type[k];
            tk.grp_first = MSIM_NONE;
            if (tk.type == MSIM_TASK_COMPUTE) {
                if (s->task_ticks[k] < 1) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: task %u lasts no tick", e, k - t0);
                tk.dur = s->task_ticks[k];
            } else if (tk.type == MSIM_TASK_INTRA) {
                if (s->task_beta[k] < 1) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: task %u has no bandwidth", e, k - t0);
                const uint64_t d = (uint64_t)s->task_ticks[k] + (s->task_bytes[k] + s->task_beta[k] - 1) / s->task_beta[k];
                if (d < 1 || d >= MSIM_NONE) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: task %u duration out of range", e, k - t0);
                tk.dur = (uint32_t)d;
            } else if (tk.type == MSIM_TASK_COLL) {
                const uint32_t cl = s->task_coll[k];
                if (cl >= ncoll || named[cl]) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: task %u names collective %u badly", e, k - t0, cl);
                named[cl] = 1;
                tk.grp_first = grp_of_coll[cl];
                const uint32_t gend = cl + 1 < ncoll ? grp_of_coll[cl + 1] : coll_grp_end;
                tk.ngrp = gend - tk.grp_first;
                uint64_t nf = 0;
                for (uint32_t gi = tk.grp_first; gi < gend; gi++) {
                    grp[gi].task = k - t0;
                    nf += (uint64_t)flows_per_conn(grp[gi]) * conns_of(grp[gi]);
                }
                tw.left = (uint32_t)nf;
            } else {
                return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: task %u has unknown type %u", e, k - t0, tk.type);
            }
            tk.pred_off = (uint32_t)tpred.size();
            tk.npred = s->task_pred_off[k + 1] - s->task_pred_off[k];
            for (uint32_t q = s->task_pred_off[k]; q < s->task_pred_off[k + 1]; q++) {
                if (s->task_pred[q] >= k - t0) return fail(out, MSIM_E_INVALID_SPEC, "experiment %u: task %u has a predecessor not before it", e, k - t0);
                tpred.push_back(s->task_pred[q]);
            }
            tasks.push_back(tk);
            task_rw.push_back(tw);
        }
    }
    const uint32_t n_task = (uint32_t)tasks.size();

    /* ---- packet spraying: every switch's equal-cost egresses toward every
     * destination host, in both climbing states (filled by the search below) */
    std::vector<uint32_t> sw_row(nn, MSIM_NONE);
    uint32_t n_sw_rows = 0;
    std::vector<uint16_t> cand_tbl;
    if (lb == MSIM_LB_SPRAY) {
        for (uint32_t n = 0; n < nn; n++)
            if (layer[n] != 0) sw_row[n] = n_sw_rows++;
        if (nn > 65536 || n_sw_rows > 32768) return fail(out, MSIM_E_LIMIT, "experiment %u: too many nodes for packet spraying", e);
        cand_tbl.assign((size_t)n_sw_rows * n_hosts * 2, 0);
    }

    /* ---- routes: reverse breadth-first search over (node, may-still-climb)
     * states from every destination, then one walk per connection */
    std::vector<std::vector<uint32_t>> by_dst(nn);
    for (uint32_t c = 0; c < conn.size(); c++) by_dst[conn[c].dst].push_back(c);
    std::vector<int32_t> dist(2 * (size_t)nn);
    std::deque<uint32_t> bfs;
    std::vector<uint32_t> cand;
    std::vector<uint64_t> load(n_ports, 0);   /* packets leaving each port */
    for (uint32_t dst = 0; dst < nn; dst++) {
        if (by_dst[dst].empty()) continue;
        std::fill(dist.begin(), dist.end(), -1);
        /* state 2n: at n, may still climb; 2n+1: at n, descending only */
        dist[2 * dst] = dist[2 * dst + 1] = 0;
        bfs.clear();
        bfs.push_back(2 * dst);
        bfs.push_back(2 * dst + 1);
        while (!bfs.empty()) {
            uint32_t st = bfs.front();
            bfs.pop_front();
            uint32_t m = st >> 1;
            bool desc = st & 1;
            for (uint32_t p = pbase[m]; p < pbase[m + 1]; p++) {
                if (!port[p].alive) continue;
                uint32_t n = port_node[port[p].peer];
                if (!desc && layer[n] < layer[m]) {          /* n climbed to m */
                    if (dist[2 * n] < 0) { dist[2 * n] = dist[st] + 1; bfs.push_back(2 * n); }
                } else if (desc && layer[n] > layer[m]) {    /* n descended to m */
                    for (uint32_t ph = 0; ph < 2; ph++)
                        if (dist[2 * n + ph] < 0) { dist[2 * n + ph] = dist[st] + 1; bfs.push_back(2 * n + ph); }
                }
            }
        }
        if (lb == MSIM_LB_SPRAY) {
            /* the candidates of the walk below, for every switch and state */
            for (uint32_t n = 0; n < nn; n++) {
                if (layer[n] == 0) continue;
                for (uint32_t st = 0; st < 2; st++) {
                    const int32_t need = dist[2 * n + st];
                    if (need < 0) continue;
                    uint32_t mask = 0;
                    for (uint32_t p = pbase[n]; p < pbase[n + 1]; p++) {
                        if (!port[p].alive) continue;
                        uint32_t m = port_node[port[p].peer];
                        if (layer[m] > layer[n] && st == 0) {
                            if (dist[2 * m] >= 0 && dist[2 * m] + 1 == need) mask |= 1u << (p - pbase[n]);
                        } else if (layer[m] < layer[n]) {
                            if (dist[2 * m + 1] >= 0 && dist[2 * m + 1] + 1 == need) mask |= 1u << (p - pbase[n]);
                        }
                    }
                    cand_tbl[((size_t)sw_row[n] * n_hosts + host_of[dst]) * 2 + st] = (uint16_t)mask;
                }
            }
        }
        for (uint32_t c : by_dst[dst]) {
            Conn &cn = conn[c];
            uint32_t node = cn.src, state = 2 * node, hop = 0, links = 0;
            if (dist[state] < 0) return fail(out, MSIM_E_UNROUTABLE, "experiment %u: connection %u (host %u -> host %u) has no path", e, c, cn.src, dst);
            while (node != dst) {
                cand.clear();
                for (uint32_t p = pbase[node]; p < pbase[node + 1]; p++) {
                    if (!port[p].alive) continue;
                    uint32_t m = port_node[port[p].peer];
                    if (layer[m] > layer[node] && !(state & 1)) {
                        if (dist[2 * m] >= 0 && dist[2 * m] + 1 == dist[state]) cand.push_back(p);
                    } else if (layer[m] < layer[node]) {
                        if (dist[2 * m + 1] >= 0 && dist[2 * m + 1] + 1 == dist[state]) cand.push_back(p);
                    }
                }
                if (cand.empty()) return fail(out, MSIM_E_UNROUTABLE, "experiment %u: connection %u stuck at node %u", e, c, node);
                uint32_t pick = cand[fmix32((uint32_t)c ^ fmix32(node ^ seed)) % cand.size()];
                if (layer[node] != 0) {
                    if (hop >= MSIM_MAX_SWITCH_HOPS) return fail(out, MSIM_E_LIMIT, "experiment %u: connection %u crosses more than %u switches", e, c, MSIM_MAX_SWITCH_HOPS);
                    cn.route |= (pick - pbase[node]) << (4 * hop);
                    hop++;
                }
                load[pick] += cn.pkts;
                cn.lat += port[pick].delay;
                uint32_t next = port_node[port[pick].peer];
                if (layer[next] < layer[node]) state = 2 * next + 1;
                else state = (state & 1) ? 2 * next + 1 : 2 * next;
                node = next;
                links++;
            }
            cn.links = links;
        }
    }

    for (uint32_t p = 0; p < n_ports; p++)
        if (load[p]) out.est_ticks = std::max<uint64_t>(out.est_ticks, (load[p] + port[p].rate - 1) / port[p].rate);

    /* ---- hosts: outgoing connections in index order, flows to receive */
    std::vector<HostRO> host(n_hosts);
    std::vector<uint32_t> n_out(n_hosts, 0), left(n_hosts, 0);
    for (auto &cn : conn) n_out[host_of[cn.src]]++;
    std::vector<uint32_t> hout(conn.size());
    uint32_t acc = 0, words = 0;
    for (uint32_t n = 0; n < nn; n++) {
        if (layer[n] != 0) continue;
        uint32_t h = host_of[n];
        host[h].port = pbase[n];
        host[h].out_off = acc;
        host[h].n_out = 0;
        host[h].rdy_off = words;
        acc += n_out[h];
        words += (n_out[h] + 31) / 32;
    }
    uint64_t n_flows = 0;
    for (uint32_t c = 0; c < conn.size(); c++) {
        Conn &cn = conn[c];
        HostRO &hr = host[host_of[cn.src]];
        cn.lidx = hr.n_out;
        hout[hr.out_off + hr.n_out++] = c;
        const uint32_t F = flows_per_conn(grp[cn.grp]);
        left[host_of[cn.dst]] += F;
        n_flows += F;
        out.est_hops += cn.pkts * cn.links;
        out.est_delivered += cn.pkts;
    }

    const uint32_t W = maxd + 1, R = maxr, nconn = (uint32_t)conn.size(), ngrp = (uint32_t)grp.size();
    out.n_flows = n_flows;
    out.n_conns = nconn;
    out.n_ports = n_ports;

    /* ---- ring layout: rings only at rate 1 on small switches, where the
     * experiment qualifies (the limits of msim_layout.h's ring format) */
    if (allow_compact && allow_ring && n_task == 0 && cc == MSIM_CC_NONE && lb == MSIM_LB_ECMP && maxr == 1 &&
        Q <= RING_MAX_Q && ngrp_fits_ring(grp) && nconn > 0) {
        uint32_t maxdeg = 1, max_out = 0, n_sw = 0;
        for (uint32_t n = 0; n < nn; n++)
            if (layer[n] != 0) { maxdeg = std::max(maxdeg, deg[n]); n_sw++; }
        for (uint32_t h = 0; h < n_hosts; h++) max_out = std::max(max_out, host[h].n_out);
        bool ok = maxdeg <= RING_MAX_DEG && max_out <= RING_MAX_PAIRS;
        for (const Conn &cn : conn) ok = ok && cn.links >= 1 && cn.links - 1 <= RING_MAX_HOPS;
        const uint32_t SB = ((n_hosts + 63) / 64) * 64;
        std::vector<uint32_t> slot(n_ports), sw_of(nn, MSIM_NONE);
        uint32_t nt = SB, k_sw = 0;
        for (uint32_t n = 0; n < nn && ok; n++) {
            if (layer[n] == 0) { slot[pbase[n]] = host_of[n]; continue; }
            if ((nt & 63) + deg[n] > 64) nt = (nt + 63) & ~63u;
            sw_of[n] = k_sw++;
            for (uint32_t q = pbase[n]; q < pbase[n + 1]; q++) slot[q] = nt++;
        }
        ok = ok && nt <= 1024;
        std::vector<uint32_t> stg;
        if (ok && !ring_staging(slot, port, n_ports, nt, stg))
            return fail(out, MSIM_E_LIMIT, "experiment %u: internal error: ring staging slots", e);
        if (ok) {
            const uint32_t S = nt - SB, NS = (nt + 63) & ~63u;
            ArenaHdr3 H{};
            H.mode = MODE_RING; H.n_flows = (uint32_t)n_flows;
            H.nt = nt; H.H = n_hosts; H.SB = SB; H.Q = Q; H.W = W; H.n_grp = ngrp; H.n_sw = n_sw;
            size_t off = align16(sizeof(ArenaHdr3));
            auto take = [&](uint32_t &field, size_t bytes) { field = (uint32_t)off; off = align16(off + bytes); };
            take(H.o_grp, sizeof(RGrp) * ngrp);
            H.rw_off = (uint32_t)off;
            take(H.o_pair, sizeof(RPair) * (size_t)max_out * SB);
            take(H.o_pdesc, 4ull * Q * S);
            take(H.o_pnxt, (size_t)Q * S);
            take(H.o_head, 64ull * n_sw);
            take(H.o_nzw, 32ull * n_sw);
            take(H.o_fw, 8ull * (S + 1));
            take(H.o_sdesc, 4ull * W * NS);
            take(H.o_dq, 8ull * RING_DQ * SB);
            H.lds_bytes = (uint32_t)off;
            take(H.o_port, sizeof(RingPort) * nt);
            take(H.o_priv, sizeof(RingPriv) * nt);
            H.bytes = (uint32_t)off;
            if (H.lds_bytes <= COMPACT_LDS_LIMIT) {
                out.arena.assign(off, 0);
                uint8_t *A = out.arena.data();
                /* flow sizes: p in every round but the last, whose chunk k holds X/N + [k < X mod N] */
                auto size_at = [](const Grp &g, uint32_t r, uint32_t pos) -> uint32_t {
                    const uint32_t T1 = (g.R - 1) * g.S;
                    if (pos < T1) return g.p;
                    const uint32_t k = ring_chunk(g.kind, g.N, r, pos - T1);
                    return g.X / g.N + (k < g.X % g.N ? 1u : 0u);
                };
                RGrp *rg = (RGrp *)(A + H.o_grp);
                for (uint32_t k = 0; k < ngrp; k++) {
                    const Grp &g = grp[k];
                    rg[k].fid_base = g.fid_base; rg[k].N = g.N; rg[k].S = g.S; rg[k].RS = g.R * g.S;
                    rg[k].p = g.p; rg[k].Xq = g.X / g.N;
                    rg[k].T = 0;
                    for (uint32_t b = 0; b < 3 * g.N; b++)
                        if (b % g.N < g.X % g.N) rg[k].T |= 1u << b;
                    rg[k].mS = (uint32_t)(((1ull << 24) + g.S - 1) / g.S);
                }
                RPair *pairs = (RPair *)(A + H.o_pair);
                for (uint32_t h = 0; h < n_hosts; h++) {
                    for (uint32_t k = 0; k < host[h].n_out; k++) {
                        const uint32_t c = hout[host[h].out_off + k];
                        const Conn &cn = conn[c];
                        const Grp &g = grp[cn.grp];
                        const uint32_t i = cn.idx, ri = i == 0 ? g.N - 1 : i - 1;
                        /* the destination's pair whose partner is this connection */
                        const uint32_t kdst = conn[g.conn_base + (i + 1) % g.N].lidx;
                        uint32_t route3 = 0;
                        for (uint32_t hop = 0; hop + 1 < cn.links; hop++)
                            route3 |= ((cn.route >> (4 * hop)) & 7u) << (3 * hop);
                        RPair &pp = pairs[(size_t)k * SB + h];
                        pp.snd = (CS_ACTIVE << 30) | size_at(g, i, 0);
                        pp.rcv = 0;
                        pp.desc = route3 | (kdst << RD_PAIR_SHIFT) | (cn.grp << RD_GRP_SHIFT) | RD_VALID;
                        pp.gi = cn.grp | (i << 10) | (ri << 20);
                    }
                }
                memset(A + H.o_head, (int)Q_EMPTY, 64ull * n_sw);
                RingPort *rp = (RingPort *)(A + H.o_port);
                RingPriv *rv = (RingPriv *)(A + H.o_priv);
                for (uint32_t q = 0; q < n_ports; q++) {
                    const PortRO &P = port[q];
                    const uint32_t sl = slot[q], fq = P.peer;
                    RingPort &r = rp[sl];
                    r.peer = slot[fq];
                    r.flags = (uint8_t)(PF_USED | (P.alive ? PF_ALIVE : 0) | (P.is_host ? PF_HOST : 0) |
                                        (P.peer_is_host ? PF_PEER_HOST : 0));
                    r.local = P.local; r.deg = P.deg; r.delay = P.delay;
                    r.stg = (uint16_t)stg[sl];
                    r.pstg = (uint16_t)stg[slot[fq]];
                    if (P.is_host) {
                        r.row = host[P.host].n_out;
                        rv[sl].mask = host[P.host].n_out == 32 ? ~0u : ((1u << host[P.host].n_out) - 1u);
                        rv[sl].tails = left[P.host];
                    } else {
                        r.row = sw_of[port_node[q]] * 8;
                        rv[sl].mask = (1u << Q) - 1u;
                    }
                }
                memcpy(A, &H, sizeof H);
                out.rw_off = H.rw_off;
                out.bytes = H.bytes;
                out.lds_bytes = H.lds_bytes;
                out.compact = true;
                out.kind = KIND_RING;
                out.nt = nt;
                return MSIM_OK;
            }
        }
    }

    /* ---- compact layout, where the experiment qualifies (no task graph, no
     * congestion control, ECMP) */
    if (allow_compact && n_task == 0 && cc == MSIM_CC_NONE && lb == MSIM_LB_ECMP) {
        uint32_t maxdeg = 1, max_out = 0, max_F = 0;
        uint64_t max_size = 0;
        for (uint32_t n = 0; n < nn; n++)
            if (layer[n] != 0) maxdeg = std::max(maxdeg, deg[n]);
        for (uint32_t h = 0; h < n_hosts; h++) max_out = std::max(max_out, host[h].n_out);
        for (const Grp &g : grp) {
            max_F = std::max(max_F, flows_per_conn(g));
            if (g.kind == GK_BCAST) max_size = std::max<uint64_t>(max_size, g.p / g.S + 1);
            else if (g.kind != GK_XFLOW) max_size = std::max<uint64_t>(max_size, std::max<uint64_t>(g.p, g.X / g.N + 1));
        }
        for (auto &cn : conn)
            if (grp[cn.grp].kind == GK_XFLOW) max_size = std::max<uint64_t>(max_size, cn.idx);
        /* thread slots: hosts first; each switch's ports consecutive inside one wavefront */
        const uint32_t SB = ((n_hosts + 63) / 64) * 64;
        std::vector<uint32_t> slot(n_ports), sw_of(nn, MSIM_NONE);
        uint32_t nt = SB, n_sw = 0;
        for (uint32_t n = 0; n < nn; n++) {
            if (layer[n] == 0) { slot[pbase[n]] = host_of[n]; continue; }
            if ((nt & 63) + deg[n] > 64) nt = (nt + 63) & ~63u;
            sw_of[n] = n_sw++;
            for (uint32_t q = pbase[n]; q < pbase[n + 1]; q++) slot[q] = nt++;
        }
        const uint32_t rsz = maxdeg <= 8 ? 8 : 16, dt = nconn <= 4096 ? 2 : 4;
        uint32_t max_ring = 0;
        bool xneed = false;      /* trees, send/recv groups or gated rings */
        for (const Grp &g : grp) {
            if (g.kind == GK_RING_AR || g.kind == GK_RING_AG) max_ring = std::max(max_ring, g.S);
            if ((g.kind == GK_BCAST || g.kind == GK_SEQ || g.kind == GK_TREE) && g.N > 65535)
                max_ring = 1u << 20;   /* too many members for CGrp.N */
            if (g.kind == GK_SEQ || g.kind == GK_TREE || g.link != MSIM_NONE) xneed = true;
        }
        const uint32_t base_kind = 1 + ((maxdeg > 8 ? 4u : 0u) | (nconn > 4096 ? 2u : 0u) | (R > 1 ? 1u : 0u));
        /* the two kernels with those rules, and their thread bound */
        const bool x_ok = !xneed || ((base_kind == 1 || base_kind == 6) && nt <= COMPACT_X_THREADS);
        if (nt <= 1024 && maxdeg <= 16 && Q <= 64 && max_out <= 64 && max_F <= C_POS_MASK && max_size < 65536 &&
            max_ring < 1024 && ngrp <= 65535 && nconn < (1u << (32 - DESC_SHIFT)) && x_ok) {
            const uint32_t S = nt - SB;                 /* switch slots, gaps included */
            const uint32_t Vc = n_sw * rsz * rsz;
            ArenaHdr2 H{};
            H.mode = MODE_COMPACT; H.n_flows = (uint32_t)n_flows;
            H.nt = nt; H.H = n_hosts; H.SB = SB;
            H.Q = Q; H.W = W; H.R = R; H.n_conn = nconn; H.n_grp = ngrp; H.rsz = rsz; H.dt = dt;
            H.flags = 0;
            if (std::all_of(grp.begin(), grp.end(), [](const Grp &g) { return g.kind == GK_RING_AR || g.kind == GK_RING_AG; }))
                H.flags |= AF_RINGS_ONLY;
            size_t off = align16(sizeof(ArenaHdr2));
            auto take = [&](uint32_t &field, size_t bytes) { field = (uint32_t)off; off = align16(off + bytes); };
            take(H.o_route, 4ull * nconn);
            take(H.o_cgrp, 2ull * nconn);
            take(H.o_lidx, (size_t)nconn);
            take(H.o_grp, sizeof(CGrp) * ngrp);
            take(H.o_hout, (size_t)dt * nconn);
            H.rw_off = (uint32_t)off;
            take(H.o_arr, Vc);
            H.o_head = 0;
            take(H.o_nslot, Vc);
            take(H.o_pdesc, (size_t)dt * S * Q);
            take(H.o_pnxt, (size_t)S * Q);
            take(H.o_popped, 8ull * nt);
            const uint32_t RP = R <= 1 ? 1 : (R <= 2 ? 2 : 4);
            H.o_elig = 0;
            take(H.o_fmask, 8ull * S);
            take(H.o_sdesc, (size_t)dt * nt * W * RP);
            take(H.o_crw, sizeof(CRW2) * nconn);
            H.lds_bytes = (uint32_t)off;
            take(H.o_port, sizeof(PortRO2) * nt);
            take(H.o_priv, sizeof(PortPriv) * nt);
            H.bytes = (uint32_t)off;
            if (H.lds_bytes <= COMPACT_LDS_LIMIT) {
                out.arena.assign(off, 0);
                uint8_t *A = out.arena.data();
                uint32_t *route = (uint32_t *)(A + H.o_route);
                uint16_t *cg = (uint16_t *)(A + H.o_cgrp);
                uint8_t *li = A + H.o_lidx;
                CRW2 *crw = (CRW2 *)(A + H.o_crw);
                for (uint32_t c = 0; c < nconn; c++) {
                    route[c] = conn[c].route;
                    cg[c] = (uint16_t)conn[c].grp;
                    li[c] = (uint8_t)conn[c].lidx;
                    const Grp &g = grp[conn[c].grp];
                    uint32_t first = first_flow_size(g, conn[c].idx);
                    crw[c].r_rem = (uint16_t)first;
                    if (g.kind == GK_XFLOW) crw[c].s_rem = (uint16_t)first;
                }
                CGrp *cgt = (CGrp *)(A + H.o_grp);
                for (uint32_t k = 0; k < ngrp; k++) {
                    const Grp &g = grp[k];
                    CGrp &o = cgt[k];
                    o.kind = (uint16_t)g.kind;
                    o.N = (uint16_t)g.N;
                    o.S = g.S;
                    o.R = g.R;
                    o.fid_base = g.fid_base;
                    o.conn_base = g.conn_base;
                    o.mS = (uint32_t)(((1ull << 24) + g.S - 1) / g.S);
                    o.link = g.link;
                    if (g.kind == GK_BCAST) { o.p = g.p / g.S; o.Xq = g.p % g.S; o.Xr = 0; }
                    else if (g.kind == GK_XFLOW) { o.p = 0; o.Xq = 0; o.Xr = 0; }
                    else if (g.kind == GK_TREE) { o.p = g.p; o.Xq = g.X; o.Xr = 0; }
                    else if (g.kind == GK_SEQ) { o.p = g.p; o.Xq = 0; o.Xr = g.X; }
                    else { o.p = g.p; o.Xq = g.X / g.N; o.Xr = g.X % g.N; }
                }
                for (uint32_t c = 0; c < nconn; c++) {
                    if (dt == 2) ((uint16_t *)(A + H.o_hout))[c] = (uint16_t)hout[c];
                    else ((uint32_t *)(A + H.o_hout))[c] = hout[c];
                }
                PortRO2 *pro = (PortRO2 *)(A + H.o_port);
                PortPriv *pv = (PortPriv *)(A + H.o_priv);
                for (uint32_t p = 0; p < n_ports; p++) {
                    const PortRO &P = port[p];
                    const uint32_t sl = slot[p];
                    PortRO2 &R2 = pro[sl];
                    R2.peer = slot[P.peer];
                    R2.rate = P.rate;
                    R2.delay = P.delay;
                    R2.local = P.local;
                    R2.deg = P.deg;
                    R2.flags = (uint8_t)(PF_USED | (P.alive ? PF_ALIVE : 0) | (P.is_host ? PF_HOST : 0) |
                                         (P.peer_is_host ? PF_PEER_HOST : 0));
                    if (P.is_host) {
                        R2.vbase = host[P.host].out_off;
                        R2.n_out = (uint16_t)host[P.host].n_out;
                        pv[sl].left = left[P.host];
                    } else {
                        R2.vbase = sw_of[port_node[p]] * rsz * rsz;
                        pv[sl].freem = Q == 64 ? ~0ull : ((1ull << Q) - 1ull);
                    }
                }
                /* every queue starts empty (head byte Q_EMPTY) */
                memset(A + H.o_nslot, (int)Q_EMPTY, Vc);
                memcpy(A, &H, sizeof H);
                out.rw_off = H.rw_off;
                out.bytes = H.bytes;
                out.lds_bytes = H.lds_bytes;
                out.compact = true;
                out.kind = 1 + ((rsz == 16 ? 4u : 0u) | (dt == 4 ? 2u : 0u) | (R > 1 ? 1u : 0u));
                if (xneed) out.kind = out.kind == 1 ? KIND_COMPACT_X8 : KIND_COMPACT_X16;
                out.nt = nt;
                return MSIM_OK;
            }
        }
    }

    /* ---- general layout */
    /* switch ports own the buffer pools; a switch port's host field gives the
     * pool index of its switch's port 0 (its own is that + its local index) */
    std::vector<PortRO> gport = port;
    uint32_t n_swp = 0;
    for (uint32_t n = 0; n < nn; n++) {
        if (layer[n] == 0) continue;
        for (uint32_t p = pbase[n]; p < pbase[n + 1]; p++) gport[p].host = n_swp;
        n_swp += deg[n];
    }
    ArenaHdr H{};
    H.mode = MODE_GENERAL;
    H.n_ports = n_ports; H.n_hosts = n_hosts; H.n_conn = nconn; H.n_grp = ngrp;
    H.Q = Q; H.W = W; H.R = R; H.n_voq = n_voq; H.n_flows = (uint32_t)n_flows;
    size_t off = align16(sizeof(ArenaHdr));
    auto take = [&](uint32_t &field, size_t bytes) { field = (uint32_t)off; off = align16(off + bytes); };
    /* read-only, touched by every port every tick: header, ports, hosts (and
     * the sprayed port info); then the per-connection tables */
    take(H.o_port, sizeof(PortRO) * n_ports);
    take(H.o_host, sizeof(HostRO) * n_hosts);
    H.lb = lb;
    H.seed = seed;
    std::vector<uint32_t> rwoff;
    if (lb == MSIM_LB_SPRAY) {
        uint64_t smax = 1;
        for (const Conn &cn : conn) smax = std::max<uint64_t>(smax, cn.pkts);
        uint32_t sbits = 1, cbits = 1;
        while ((1ull << sbits) < smax) sbits++;
        while ((1ull << cbits) < nconn) cbits++;
        if (sbits + cbits > 32) return fail(out, MSIM_E_LIMIT, "experiment %u: connections x packets too large for sprayed descriptors", e);
        H.sbits = sbits;
        take(H.o_spi, 4ull * n_ports);
    }
    H.ro_hot = (uint32_t)off;
    take(H.o_conn, sizeof(ConnRO) * nconn);
    take(H.o_grp, sizeof(Grp) * ngrp);
    take(H.o_hout, 4ull * nconn);
    H.n_task = n_task;
    take(H.o_task, sizeof(TaskRO) * n_task);
    take(H.o_tpred, 4ull * tpred.size());
    if (lb == MSIM_LB_SPRAY) {
        take(H.o_cand, 2ull * cand_tbl.size());
        rwoff.assign(nconn + 1, 0);
        for (uint32_t c = 0; c < nconn; c++) rwoff[c + 1] = rwoff[c] + (uint32_t)((conn[c].pkts + 31) / 32);
        take(H.o_rwoff, 4ull * (nconn + 1));
    }
    H.rw_off = (uint32_t)off;
    take(H.o_tail, n_voq);
    take(H.o_nslot, n_voq);
    take(H.o_fmask, 32ull * n_swp);
    take(H.o_ow, 4ull * n_ports);
    take(H.o_pdesc, 4ull * n_swp * Q);
    take(H.o_pnxt, (size_t)n_swp * Q);
    take(H.o_pstate, sizeof(PortRW) * n_ports);
    take(H.o_scnt, (size_t)n_ports * W);
    take(H.o_sdesc, 4ull * n_ports * W * R);
    H.cc = cc;
    H.ecn_k = ecn_k;
    H.WA = 1;
    H.n_rdy = words;
    /* HPCC: telemetry records of up to hx switches, one per packet in flight
     * (the window never exceeds T = 2 L packets), found from the descriptor */
    H.cshift = DESC_SHIFT;
    uint64_t int_records = 0;
    if (cc == MSIM_CC_HPCC) {
        uint32_t smax = 1;
        for (const Conn &cn : conn) {
            H.hx = std::max(H.hx, cn.links - 1);
            smax = std::max(smax, 2 * cn.lat);
            int_records += 2ull * cn.lat;
        }
        uint32_t sb = 0;
        while ((1u << sb) < smax) sb++;
        H.cshift = 4 + sb;
        if (H.cshift >= 31 || (uint64_t)nconn > (1ull << (31 - H.cshift)))
            return fail(out, MSIM_E_LIMIT, "experiment %u: too many connections for HPCC descriptors", e);
    }
    if (cc != MSIM_CC_NONE) {
        uint32_t max_lat = 0;
        for (const Conn &cn : conn) max_lat = std::max(max_lat, cn.lat);
        while (H.WA <= max_lat) H.WA <<= 1;
        take(H.o_bl, 4ull * n_ports);
        take(H.o_qlen, 4ull * n_ports);
        take(H.o_ackm, 4ull * H.WA * words);
    }
    take(H.o_hstate, sizeof(HostRW) * n_hosts);
    take(H.o_hpc, n_hosts);
    take(H.o_ready, 4ull * words);
    /* [rw_off, rw_hot) with [0, ro_hot): the state of the switch and NIC phases,
     * placed in LDS on its own when the whole arena does not fit */
    H.rw_hot = (uint32_t)off;
    take(H.o_cstate, sizeof(ConnRW) * nconn);
    take(H.o_trw, sizeof(TaskRW) * n_task);
    if (cc != MSIM_CC_NONE) {
        take(H.o_cc, sizeof(CcRW) * nconn);
        take(H.o_ack, 2ull * nconn * H.WA);
    }
    if (cc == MSIM_CC_HPCC) {
        take(H.o_hl, 12ull * H.hx * nconn);
        take(H.o_int, 12ull * H.hx * int_records);
    }
    if (lb == MSIM_LB_SPRAY) {
        take(H.o_sseq, 4ull * nconn);
        take(H.o_rnext, 4ull * nconn);
        take(H.o_rbits, 4ull * rwoff[nconn]);
    }
    if (off > 0xFFFFFFF0ull) return fail(out, MSIM_E_LIMIT, "experiment %u: state of %zu bytes too large", e, off);
    H.bytes = (uint32_t)off;
    {
        /* the kernel addresses the switch and NIC state as LDS and the rest as
         * global memory when only the former fits in LDS, taking each array's
         * side from this order: check that every array lies on its side */
        const uint64_t hot_lo[2] = {0, H.rw_off}, hot_hi[2] = {H.ro_hot, H.rw_hot};
        auto within = [&](uint32_t o, uint64_t bytes, bool hot) {
            if (bytes == 0) return true;
            const bool in0 = o >= hot_lo[0] && o + bytes <= hot_hi[0], in1 = o >= hot_lo[1] && o + bytes <= hot_hi[1];
            const bool out0 = o + bytes <= hot_lo[0] || o >= hot_hi[0], out1 = o + bytes <= hot_lo[1] || o >= hot_hi[1];
            return hot ? (in0 || in1) : (out0 && out1);
        };
        const uint64_t WA = H.WA;
        const bool ok = within(H.o_port, sizeof(PortRO) * n_ports, true) && within(H.o_host, sizeof(HostRO) * n_hosts, true) &&
            within(H.o_spi, lb == MSIM_LB_SPRAY ? 4ull * n_ports : 0, true) &&
            within(H.o_tail, n_voq, true) && within(H.o_nslot, n_voq, true) && within(H.o_fmask, 32ull * n_swp, true) &&
            within(H.o_ow, 4ull * n_ports, true) && within(H.o_pdesc, 4ull * n_swp * Q, true) &&
            within(H.o_pnxt, (uint64_t)n_swp * Q, true) && within(H.o_pstate, sizeof(PortRW) * n_ports, true) &&
            within(H.o_scnt, (uint64_t)n_ports * W, true) && within(H.o_sdesc, 4ull * n_ports * W * R, true) &&
            within(H.o_bl, cc != MSIM_CC_NONE ? 4ull * n_ports : 0, true) &&
            within(H.o_qlen, cc != MSIM_CC_NONE ? 4ull * n_ports : 0, true) &&
            within(H.o_ackm, cc != MSIM_CC_NONE ? 4ull * WA * words : 0, true) &&
            within(H.o_hstate, sizeof(HostRW) * n_hosts, true) && within(H.o_hpc, n_hosts, true) &&
            within(H.o_ready, 4ull * words, true) &&
            within(H.o_conn, sizeof(ConnRO) * nconn, false) && within(H.o_grp, sizeof(Grp) * ngrp, false) &&
            within(H.o_hout, 4ull * nconn, false) && within(H.o_task, sizeof(TaskRO) * n_task, false) &&
            within(H.o_tpred, 4ull * tpred.size(), false) && within(H.o_cstate, sizeof(ConnRW) * nconn, false) &&
            within(H.o_trw, sizeof(TaskRW) * n_task, false) &&
            within(H.o_cc, cc != MSIM_CC_NONE ? sizeof(CcRW) * nconn : 0, false) &&
            within(H.o_ack, cc != MSIM_CC_NONE ? 2ull * nconn * WA : 0, false) &&
            within(H.o_hl, cc == MSIM_CC_HPCC ? 12ull * H.hx * nconn : 0, false) &&
            within(H.o_int, cc == MSIM_CC_HPCC ? 12ull * H.hx * int_records : 0, false) &&
            within(H.o_cand, lb == MSIM_LB_SPRAY ? 2ull * cand_tbl.size() : 0, false) &&
            within(H.o_rwoff, lb == MSIM_LB_SPRAY ? 4ull * (nconn + 1) : 0, false) &&
            within(H.o_sseq, lb == MSIM_LB_SPRAY ? 4ull * nconn : 0, false) &&
            within(H.o_rnext, lb == MSIM_LB_SPRAY ? 4ull * nconn : 0, false) &&
            within(H.o_rbits, lb == MSIM_LB_SPRAY ? 4ull * rwoff[nconn] : 0, false);
        if (!ok) return fail(out, MSIM_E_LIMIT, "experiment %u: internal error: general layout order", e);
    }
    out.arena.assign(off, 0);
    uint8_t *A = out.arena.data();
    memcpy(A, &H, sizeof H);
    memcpy(A + H.o_port, gport.data(), sizeof(PortRO) * n_ports);
    std::vector<ConnRO> cro(nconn);
    for (uint32_t c = 0; c < nconn; c++)   /* sprayed: the route field holds the destination host */
        cro[c] = ConnRO{lb == MSIM_LB_SPRAY ? host_of[conn[c].dst] : conn[c].route, conn[c].grp, conn[c].idx, conn[c].lidx};
    if (lb == MSIM_LB_SPRAY) {
        uint32_t *spi = (uint32_t *)(A + H.o_spi);
        for (uint32_t p = 0; p < n_ports; p++) {
            const uint32_t n = port_node[p];
            if (layer[n] == 0) continue;
            const bool from_above = layer[port_node[port[p].peer]] > layer[n];
            spi[p] = n | (sw_row[n] << 16) | (from_above ? 0x80000000u : 0u);
        }
        memcpy(A + H.o_cand, cand_tbl.data(), 2ull * cand_tbl.size());
        memcpy(A + H.o_rwoff, rwoff.data(), 4ull * (nconn + 1));
    }
    if (nconn) memcpy(A + H.o_conn, cro.data(), sizeof(ConnRO) * nconn);
    if (ngrp) memcpy(A + H.o_grp, grp.data(), sizeof(Grp) * ngrp);
    if (nconn) memcpy(A + H.o_hout, hout.data(), 4ull * nconn);
    if (n_hosts) memcpy(A + H.o_host, host.data(), sizeof(HostRO) * n_hosts);
    /* every queue starts empty, every buffer slot free */
    memset(A + H.o_nslot, (int)Q_EMPTY, n_voq);
    for (uint32_t p = 0; p < n_ports; p++) {
        if (port[p].is_host) continue;
        uint64_t *fm = (uint64_t *)(A + H.o_fmask) + 4ull * (gport[p].host + gport[p].local);
        for (uint32_t k = 0; k < Q; k++) fm[k >> 6] |= 1ull << (k & 63);
    }
    ConnRW *cs = (ConnRW *)(A + H.o_cstate);
    for (uint32_t c = 0; c < nconn; c++) cs[c].r_rem = first_flow_size(grp[conn[c].grp], conn[c].idx);
    HostRW *hs = (HostRW *)(A + H.o_hstate);
    for (uint32_t h = 0; h < n_hosts; h++) hs[h].left = left[h];
    if (cc != MSIM_CC_NONE) {
        CcRW *cr = (CcRW *)(A + H.o_cc);
        QcnRW *qr = (QcnRW *)(A + H.o_cc);
        HpRW *hr = (HpRW *)(A + H.o_cc);
        uint32_t int_off = 0;
        for (uint32_t c = 0; c < nconn; c++) {
            const uint32_t aword = host[host_of[conn[c].src]].rdy_off + (conn[c].lidx >> 5);
            if (cc == MSIM_CC_DCTCP) {
                cr[c] = CcRW{};
                cr[c].cwnd = cwnd0 << 8;
                cr[c].alpha = 1024;
                cr[c].lat = conn[c].lat;
                cr[c].aword = aword;
            } else if (cc == MSIM_CC_HPCC) {
                hr[c] = HpRW{};
                hr[c].T = hr[c].slots = 2 * conn[c].lat;
                hr[c].w = hr[c].wc = hr[c].T << 8;
                hr[c].wai = std::max(1u, (uint32_t)((uint64_t)hr[c].T * 256u * (65536u - HP_ETA) / (65536ull * HP_N)));
                hr[c].lat = conn[c].lat;
                hr[c].aword = aword;
                hr[c].nsw = conn[c].links - 1;
                hr[c].int_off = int_off;
                int_off += hr[c].slots;
            } else {
                qr[c] = QcnRW{};
                qr[c].rc = qr[c].rt = QCN_ONE;
                qr[c].alpha = 1024;
                qr[c].last_cnp = MSIM_NONE;
                qr[c].next_inc = qr[c].next_alpha = QCN_PERIOD;
                qr[c].lat = conn[c].lat;
                qr[c].aword = aword;
            }
        }
    }
    if (n_task) {
        memcpy(A + H.o_task, tasks.data(), sizeof(TaskRO) * n_task);
        if (!tpred.empty()) memcpy(A + H.o_tpred, tpred.data(), 4ull * tpred.size());
        memcpy(A + H.o_trw, task_rw.data(), sizeof(TaskRW) * n_task);
    }
    out.n_task = n_task;
    out.o_trw = H.o_trw;
    out.kind = cc != MSIM_CC_NONE ? KIND_GENERAL_CC : lb == MSIM_LB_SPRAY ? KIND_GENERAL_SPRAY
             : n_task ? KIND_GENERAL_TASKS : 0;
    out.rw_off = H.rw_off;
    out.bytes = H.bytes;
    out.split_bytes = H.ro_hot + (H.rw_hot - H.rw_off);
    out.port_bytes = (uint32_t)align16(sizeof(PortRO) * n_ports);
    return MSIM_OK;
}

} // namespace

struct msim_ctx {
    uint32_t n_exp = 0;
    std::vector<Compiled> exps;
    std::vector<uint32_t> order;
    std::vector<uint64_t> arena_off, pristine_off, rec_off;
    std::vector<uint8_t> recorded;
    uint64_t o_state = 0, o_arena_off = 0, o_order = 0, o_rec_off = 0, o_pristine = 0, o_rec_all = 0;
    uint64_t rec_words = 0, ws_bytes = 0;
    uint32_t block = 0, grid = 0, lds = 0, n_lds = 0, max_ports = 0, force_global = 0;
    uint32_t k_base[MSIM_KINDS] = {}, k_count[MSIM_KINDS] = {}, k_block[MSIM_KINDS] = {};
    uint32_t k_grid[MSIM_KINDS] = {}, k_lds[MSIM_KINDS] = {};
    uint64_t max_arena = 0;
    uint64_t max_exp_hops = 0;   /* largest packet-hop total of one experiment */
    uint8_t *ws = nullptr;
    bool bound = false;
    std::string err;
    msim_info info{};
};

static int ctx_fail(msim_ctx *c, int code, const std::string &m)
{
    if (c) c->err = m;
    return code;
}

static int hip_fail(msim_ctx *c, hipError_t e, const char *what)
{
    return ctx_fail(c, MSIM_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

extern "C" int msim_create(const msim_batch_spec *spec, const msim_options *opts, msim_ctx **out)
{
    g_create_error.clear();
    if (!out) { g_create_error = "null output pointer"; return MSIM_E_ARG; }
    *out = nullptr;
    if (!spec) { g_create_error = "null spec"; return MSIM_E_ARG; }
    if (spec->version != MSIM_ABI_VERSION) { g_create_error = "spec version mismatch"; return MSIM_E_ARG; }
    if (opts && opts->version != MSIM_ABI_VERSION) { g_create_error = "options version mismatch"; return MSIM_E_ARG; }
    const uint32_t E = spec->n_exp;
    if (E == 0 || !spec->exp_topo || !spec->exp_work || !spec->exp_queue_pkts || !spec->exp_ecmp_seed ||
        !spec->exp_pkt_bytes || !spec->topo_node_off || !spec->topo_cable_off || !spec->work_coll_off ||
        !spec->work_xflow_off) {
        g_create_error = "empty batch or missing array";
        return MSIM_E_ARG;
    }
    msim_ctx *ctx = new msim_ctx();
    ctx->n_exp = E;
    ctx->exps.resize(E);
    ctx->force_global = opts ? opts->force_global : 0;
    unsigned nt = opts && opts->host_threads ? opts->host_threads : std::max(1u, std::thread::hardware_concurrency());
    nt = std::min<unsigned>(nt, E);
    std::atomic<uint32_t> next{0};
    auto worker = [&]() {
        for (;;) {
            uint32_t e = next.fetch_add(1);
            if (e >= E) break;
            compile_exp(spec, e, !ctx->force_global, !(opts && opts->no_ring_path), ctx->exps[e]);
        }
    };
    std::vector<std::thread> th;
    for (unsigned i = 1; i < nt; i++) th.emplace_back(worker);
    worker();
    for (auto &x : th) x.join();
    for (uint32_t e = 0; e < E; e++)
        if (ctx->exps[e].err) {
            g_create_error = ctx->exps[e].msg;
            int code = ctx->exps[e].err;
            delete ctx;
            return code;
        }
    /* recorded experiments */
    ctx->recorded.assign(E, 0);
    if (opts && opts->n_record) {
        if (!opts->record_exp) { g_create_error = "record_exp is null"; delete ctx; return MSIM_E_ARG; }
        for (uint32_t i = 0; i < opts->n_record; i++) {
            if (opts->record_exp[i] >= E) { g_create_error = "record_exp index out of range"; delete ctx; return MSIM_E_ARG; }
            ctx->recorded[opts->record_exp[i]] = 1;
        }
    }
    /* longest-processing-time order: the longest experiments are claimed
     * first, by an estimate of their duration: the busiest link's load (a
     * bound on the ticks), then packet-hops.  A ring-format tick costs more
     * the smaller the chunks, each chunk's end being a flow's completion and
     * the next one's start at every rank: measured on the k=8 fat-tree
     * batch, about 1,058 + 5,400 / p cycles per tick for chunks of p
     * packets, so those experiments weigh their load by (p + 4) / p for
     * their smallest chunk (duration correlation 0.95 against 0.89 for the
     * load alone).  The general path walks every port every tick, so its
     * tick costs about the port count (on the k=16 fat-tree batch, 2.4e-8 s
     * per port-tick at every oversubscription): those experiments weigh their
     * load by their ports.  A compact tick costs about the same whatever the
     * experiment (one thread per port) */
    auto est = [](const Compiled &c) -> uint64_t {
        if (c.kind == KIND_RING && c.ring_pmin) return c.est_ticks * (c.ring_pmin + 4) / c.ring_pmin;
        if (!c.compact && c.kind != KIND_RING) return c.est_ticks * c.n_ports;
        return c.est_ticks;
    };
    ctx->order.resize(E);
    for (uint32_t e = 0; e < E; e++) ctx->order[e] = e;
    std::stable_sort(ctx->order.begin(), ctx->order.end(), [&](uint32_t a, uint32_t b) {
        const Compiled &x = ctx->exps[a], &y = ctx->exps[b];
        if (x.kind != y.kind) return x.kind < y.kind;
        const uint64_t ex = est(x), ey = est(y);
        if (ex != ey) return ex > ey;
        return x.est_hops > y.est_hops;
    });
    for (uint32_t i = 0; i < E; i++) {
        uint32_t k = ctx->exps[ctx->order[i]].kind;
        if (ctx->k_count[k] == 0) ctx->k_base[k] = i;
        ctx->k_count[k]++;
    }
    /* workspace layout */
    uint64_t off = 256;
    auto take = [&](uint64_t bytes) { uint64_t o = off; off = (off + bytes + 255) & ~255ull; return o; };
    ctx->o_state = take(sizeof(ExpState) * (uint64_t)E);
    ctx->o_arena_off = take(8ull * E);
    ctx->o_order = take(4ull * E);
    ctx->o_rec_off = take(8ull * E);
    ctx->o_pristine = take(8ull * E);
    ctx->arena_off.resize(E);
    ctx->pristine_off.resize(E);
    ctx->rec_off.assign(E, ~0ull);
    msim_info &I = ctx->info;
    for (uint32_t e = 0; e < E; e++) {
        const Compiled &c = ctx->exps[e];
        ctx->arena_off[e] = take(c.bytes);
        ctx->max_arena = std::max<uint64_t>(ctx->max_arena, c.bytes);
        ctx->max_ports = std::max<uint32_t>(ctx->max_ports, (uint32_t)c.n_ports);
        I.total_flows += c.n_flows;
        I.total_conns += c.n_conns;
        I.est_pkt_hops += c.est_hops;
        ctx->max_exp_hops = std::max(ctx->max_exp_hops, c.est_hops);
        I.est_delivered += c.est_delivered;
    }
    for (uint32_t e = 0; e < E; e++) ctx->pristine_off[e] = take(ctx->exps[e].bytes - ctx->exps[e].rw_off);
    ctx->o_rec_all = off;
    uint64_t rw = 0;
    for (uint32_t e = 0; e < E; e++)
        if (ctx->recorded[e]) { ctx->rec_off[e] = off + 4ull * rw; rw += 3ull * ctx->exps[e].n_flows; }
    ctx->rec_words = rw;
    take(4ull * rw);
    ctx->ws_bytes = off;
    /* every region a kernel touches must lie inside the workspace */
    bool inside = ctx->o_pristine + 8ull * E <= ctx->arena_off[0] && ctx->o_rec_all + 4ull * rw <= off;
    for (uint32_t e = 0; e < E && inside; e++) {
        const Compiled &c = ctx->exps[e];
        inside = ctx->arena_off[e] + c.bytes <= ctx->pristine_off[0] &&
                 ctx->pristine_off[e] + (c.bytes - c.rw_off) <= ctx->o_rec_all &&
                 (!ctx->recorded[e] || ctx->rec_off[e] + 12ull * c.n_flows <= off);
    }
    if (!inside) { g_create_error = "internal error: workspace layout overlaps its bounds"; delete ctx; return MSIM_E_LIMIT; }
    /* launch shape per kernel kind: a compact experiment needs one thread per
     * port slot; the general path strides its threads over the ports */
    for (uint32_t e = 0; e < E; e++) {
        const Compiled &c = ctx->exps[e];
        uint32_t need = c.compact ? c.nt : std::min<uint32_t>(kind_max_threads(c.kind), (uint32_t)c.n_ports);
        ctx->k_block[c.kind] = std::max(ctx->k_block[c.kind], ((need + 63) / 64) * 64);
        if (c.compact) I.n_compact++;
    }
    for (uint32_t k = 0; k < MSIM_KINDS; k++) {
        if (!ctx->k_count[k]) continue;
        uint32_t bt = std::max(64u, ctx->k_block[k]);
        if (opts && opts->block_threads) {
            bt = opts->block_threads;
            const bool general = k == 0 || k == KIND_GENERAL_TASKS || k == KIND_GENERAL_CC || k == KIND_GENERAL_SPRAY;
            if (bt % 64 || bt > kind_max_threads(k) || bt < 64 || (!general && bt < ctx->k_block[k])) {
                g_create_error = "block_threads must be a multiple of 64 within the kernel's launch bound, covering every compact experiment's ports";
                delete ctx;
                return MSIM_E_ARG;
            }
        }
        ctx->k_block[k] = bt;
    }
    uint32_t main_kind = 0;
    for (uint32_t k = 0; k < MSIM_KINDS; k++)
        if (ctx->k_count[k] > ctx->k_count[main_kind]) main_kind = k;
    ctx->block = ctx->k_block[main_kind];
    I.main_kernel = main_kind;
    const uint32_t bt = ctx->block;
    I.n_exp = E;
    I.block_threads = bt;
    I.max_ports = ctx->max_ports;
    I.max_arena_bytes = ctx->max_arena;
    I.workspace_bytes = ctx->ws_bytes;
    *out = ctx;
    return MSIM_OK;
}

extern "C" int msim_workspace_size(const msim_ctx *ctx, uint64_t *bytes)
{
    if (!ctx || !bytes) return MSIM_E_ARG;
    *bytes = ctx->ws_bytes;
    return MSIM_OK;
}

extern "C" int msim_bind(msim_ctx *ctx, void *dev_ws, uint64_t ws_bytes, void *stream_)
{
    if (!ctx) return MSIM_E_ARG;
    hipStream_t stream = (hipStream_t)stream_;
    if (!dev_ws || ws_bytes < ctx->ws_bytes || ((uintptr_t)dev_ws & 255))
        return ctx_fail(ctx, MSIM_E_WORKSPACE, "workspace missing, smaller than msim_workspace_size or not 256-byte aligned");
    ctx->ws = (uint8_t *)dev_ws;
    const uint32_t E = ctx->n_exp;
    /* LDS placement: every arena that fits in the LDS a workgroup can get */
    int dev = 0, max_lds = 0, n_cu = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he == hipSuccess) he = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (he == hipSuccess) he = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (he != hipSuccess) return hip_fail(ctx, he, "device query");
    const uint32_t static_lds = 4096;
    uint32_t budget = max_lds > (int)static_lds ? (uint32_t)max_lds - static_lds : 0;
    ctx->n_lds = 0;
    uint32_t main_kind = 0;
    for (uint32_t k = 0; k < MSIM_KINDS; k++) {
        ctx->k_lds[k] = 0;
        ctx->k_grid[k] = 0;
        if (ctx->k_count[k] > ctx->k_count[main_kind]) main_kind = k;
    }
    for (uint32_t e = 0; e < E; e++) {
        const Compiled &c = ctx->exps[e];
        if (c.compact) {
            if (c.lds_bytes > budget)
                return ctx_fail(ctx, MSIM_E_LIMIT, "device LDS too small for a compact experiment");
            ctx->k_lds[c.kind] = std::max(ctx->k_lds[c.kind], c.lds_bytes);
            ctx->n_lds++;
        } else if (!ctx->force_global && c.bytes <= budget) {
            ctx->k_lds[c.kind] = std::max(ctx->k_lds[c.kind], c.bytes);
            ctx->n_lds++;
        } else if (!ctx->force_global && c.split_bytes && c.split_bytes <= budget) {
            ctx->k_lds[c.kind] = std::max(ctx->k_lds[c.kind], c.split_bytes);   /* switch/NIC state only */
            ctx->n_lds++;
        } else if (!ctx->force_global && c.port_bytes && c.port_bytes <= budget) {
            ctx->k_lds[c.kind] = std::max(ctx->k_lds[c.kind], c.port_bytes);    /* the port table only */
        }
    }
    for (uint32_t k = 0; k < MSIM_KINDS; k++) {
        if (!ctx->k_count[k]) continue;
        uint32_t l = ctx->k_lds[k] ? ((ctx->k_lds[k] + 255) / 256) * 256 : 0;
        if (l > budget) l = ctx->k_lds[k];
        ctx->k_lds[k] = l;
        if (l) {
            he = msim_set_lds_limit(k, l);
            if (he != hipSuccess) return hip_fail(ctx, he, "hipFuncSetAttribute(dynamic LDS)");
        }
        int per_cu = 0;
        he = msim_occupancy(k, ctx->k_block[k], l, &per_cu);
        if (he != hipSuccess) return hip_fail(ctx, he, "occupancy query");
        if (per_cu < 1) per_cu = 1;
        ctx->k_grid[k] = (uint32_t)std::min<uint64_t>(ctx->k_count[k], (uint64_t)n_cu * per_cu);
    }
    ctx->lds = ctx->k_lds[main_kind];
    ctx->grid = ctx->k_grid[main_kind];
    ctx->info.grid_blocks = ctx->grid;
    ctx->info.lds_bytes = ctx->lds;
    ctx->info.n_lds_exp = ctx->n_lds;
    /* upload: tables, then arenas and their pristine mutable parts */
    std::vector<uint8_t> head(ctx->exps.empty() ? 0 : (size_t)(ctx->arena_off[0]), 0);
    WsHdr wh{};
    wh.n_exp = E;
    memcpy(head.data(), &wh, sizeof wh);
    ExpState *st = (ExpState *)(head.data() + ctx->o_state);
    for (uint32_t e = 0; e < E; e++) {
        st[e] = ExpState{};
        st[e].status = ctx->exps[e].n_flows == 0 ? MSIM_EXP_DONE : MSIM_EXP_INCOMPLETE;
    }
    memcpy(head.data() + ctx->o_arena_off, ctx->arena_off.data(), 8ull * E);
    memcpy(head.data() + ctx->o_order, ctx->order.data(), 4ull * E);
    memcpy(head.data() + ctx->o_rec_off, ctx->rec_off.data(), 8ull * E);
    memcpy(head.data() + ctx->o_pristine, ctx->pristine_off.data(), 8ull * E);
    he = hipMemcpyAsync(ctx->ws, head.data(), head.size(), hipMemcpyHostToDevice, stream);
    /* arenas are contiguous in experiment order: copy them in large batches */
    std::vector<uint8_t> stage;
    auto flush = [&](uint64_t dst) -> hipError_t {
        if (stage.empty()) return hipSuccess;
        hipError_t r = hipMemcpyAsync(ctx->ws + dst, stage.data(), stage.size(), hipMemcpyHostToDevice, stream);
        if (r == hipSuccess) r = hipStreamSynchronize(stream);
        stage.clear();
        return r;
    };
    const size_t chunk = 64u << 20;
    uint64_t run_start = ctx->arena_off[0];
    for (uint32_t e = 0; e < E && he == hipSuccess; e++) {
        if (ctx->arena_off[e] != run_start + stage.size()) {
            he = flush(run_start);
            run_start = ctx->arena_off[e];
        }
        stage.insert(stage.end(), ctx->exps[e].arena.begin(), ctx->exps[e].arena.end());
        stage.resize(((stage.size() + 255) / 256) * 256, 0);
        if (stage.size() >= chunk) { he = flush(run_start); run_start = e + 1 < E ? ctx->arena_off[e + 1] : 0; }
    }
    if (he == hipSuccess) he = flush(run_start);
    if (E) run_start = ctx->pristine_off[0];
    for (uint32_t e = 0; e < E && he == hipSuccess; e++) {
        const Compiled &c = ctx->exps[e];
        if (ctx->pristine_off[e] != run_start + stage.size()) {
            he = flush(run_start);
            run_start = ctx->pristine_off[e];
        }
        stage.insert(stage.end(), c.arena.begin() + c.rw_off, c.arena.end());
        stage.resize(((stage.size() + 255) / 256) * 256, 0);
        if (stage.size() >= chunk) { he = flush(run_start); run_start = e + 1 < E ? ctx->pristine_off[e + 1] : 0; }
    }
    if (he == hipSuccess) he = flush(run_start);
    if (he == hipSuccess) he = hipStreamSynchronize(stream);
    if (he != hipSuccess) return hip_fail(ctx, he, "upload");
    ctx->bound = true;
    int rc = msim_reset(ctx, stream_);
    if (rc) return rc;
    he = hipStreamSynchronize(stream);
    if (he != hipSuccess) return hip_fail(ctx, he, "reset");
    return MSIM_OK;
}

static KParams make_params(const msim_ctx *ctx, uint32_t max_ticks)
{
    KParams kp{};
    kp.ws = ctx->ws;
    kp.o_state = ctx->o_state;
    kp.o_arena_off = ctx->o_arena_off;
    kp.o_order = ctx->o_order;
    kp.o_rec_off = ctx->o_rec_off;
    kp.o_pristine = ctx->o_pristine;
    kp.n_exp = ctx->n_exp;
    kp.max_ticks = max_ticks;
    kp.lds_bytes = ctx->lds;
    return kp;
}

/* The launches of one msim_run call.  The kernels count a port's packet-hops
 * of one launch in 32 bits.  A port never sends more than its experiment's
 * packet-hop total, so one launch per kernel kind suffices unless an
 * experiment reaches 2^32 packet-hops; then launches of at most 2^30 ticks
 * keep every port (rate <= 4) below 2^32 per launch.  claim_base == NULL: the
 * queue counters are the workspace header's, one per kind, zeroed before each
 * round of launches; otherwise launch i takes claim_base[i], all zeroed once
 * before the first launch. */
static int run_launches(msim_ctx *ctx, uint32_t max_ticks, hipStream_t stream, uint32_t *claim_base)
{
    const uint64_t step = ctx->max_exp_hops < (1ull << 32) ? max_ticks : MSIM_LAUNCH_TICKS;
    uint32_t launch = 0;
    for (uint64_t left = max_ticks; left > 0;) {
        const uint32_t chunk = (uint32_t)(left > step ? step : left);
        left -= chunk;
        bool first = true;
        for (uint32_t k = 0; k < MSIM_KINDS; k++) {
            if (!ctx->k_count[k]) continue;
            KParams kp = make_params(ctx, chunk);
            kp.order_base = ctx->k_base[k];
            kp.n_run = ctx->k_count[k];
            kp.lds_bytes = ctx->k_lds[k];
            uint32_t *clear = nullptr, n_clear = 0;
            if (claim_base) {
                kp.claim = claim_base + launch;
                if (launch == 0) { clear = claim_base; n_clear = MSIM_SCRATCH_WORDS; }
            } else {
                kp.claim = ((WsHdr *)ctx->ws)->claim + k;
                if (first) { clear = ((WsHdr *)ctx->ws)->claim; n_clear = MSIM_KINDS; }
            }
            hipError_t he = msim_launch_run(&kp, k, ctx->k_grid[k], ctx->k_block[k], ctx->k_lds[k], clear, n_clear,
                                            stream);
            if (he != hipSuccess) return hip_fail(ctx, he, "kernel launch");
            first = false;
            launch++;
        }
    }
    return MSIM_OK;
}

/* Number of kernel launches msim_run(max_ticks) makes. */
static uint64_t n_launches(const msim_ctx *ctx, uint32_t max_ticks)
{
    const uint64_t step = ctx->max_exp_hops < (1ull << 32) ? max_ticks : MSIM_LAUNCH_TICKS;
    uint64_t kinds = 0;
    for (uint32_t k = 0; k < MSIM_KINDS; k++) kinds += ctx->k_count[k] ? 1 : 0;
    const uint64_t chunks = max_ticks == 0 ? 0 : (max_ticks + step - 1) / step;
    return chunks * kinds;
}

extern "C" int msim_run(msim_ctx *ctx, uint32_t max_ticks, void *stream, uint32_t flags)
{
    if (!ctx) return MSIM_E_ARG;
    if (!ctx->bound) return ctx_fail(ctx, MSIM_E_STATE, "msim_run before msim_bind");
    (void)flags;
    return run_launches(ctx, max_ticks, (hipStream_t)stream, nullptr);
}

extern "C" int msim_run_noalloc(msim_ctx *ctx, uint32_t max_ticks, void *stream, uint32_t flags)
{
    if (!ctx) return MSIM_E_ARG;
    if (!ctx->bound) return ctx_fail(ctx, MSIM_E_STATE, "msim_run_noalloc before msim_bind");
    (void)flags;
    const uint64_t n = n_launches(ctx, max_ticks);
    if (n > MSIM_SCRATCH_WORDS)
        return ctx_fail(ctx, MSIM_E_LIMIT, "msim_run_noalloc: the call needs " + std::to_string(n) +
                                           " kernel launches; its static queue counters hold " +
                                           std::to_string(MSIM_SCRATCH_WORDS) + " (use msim_run or fewer max_ticks)");
    uint32_t *words = nullptr;
    hipError_t he = msim_scratch_words(&words);
    if (he != hipSuccess) return hip_fail(ctx, he, "scratch symbol address");
    return run_launches(ctx, max_ticks, (hipStream_t)stream, words);
}

extern "C" int msim_reset(msim_ctx *ctx, void *stream)
{
    if (!ctx) return MSIM_E_ARG;
    if (!ctx->bound) return ctx_fail(ctx, MSIM_E_STATE, "msim_reset before msim_bind");
    KParams kp = make_params(ctx, 0);
    hipError_t he = msim_launch_reset(&kp, ctx->o_rec_all, ctx->rec_words, (hipStream_t)stream);
    if (he != hipSuccess) return hip_fail(ctx, he, "reset launch");
    return MSIM_OK;
}

extern "C" int msim_results(msim_ctx *ctx, void *stream, uint8_t *exp_status, uint32_t *exp_tick,
                            uint64_t *exp_pkt_hops, uint64_t *exp_delivered, uint64_t *exp_digest)
{
    if (!ctx) return MSIM_E_ARG;
    if (!ctx->bound) return ctx_fail(ctx, MSIM_E_STATE, "msim_results before msim_bind");
    hipError_t he = hipStreamSynchronize((hipStream_t)stream);
    std::vector<ExpState> st(ctx->n_exp);
    if (he == hipSuccess) he = hipMemcpy(st.data(), ctx->ws + ctx->o_state, sizeof(ExpState) * st.size(), hipMemcpyDeviceToHost);
    if (he != hipSuccess) return hip_fail(ctx, he, "results copy");
    bool dead = false, inc = false, fault = false;
    for (uint32_t e = 0; e < ctx->n_exp; e++) {
        if (exp_status) exp_status[e] = (uint8_t)st[e].status;
        if (exp_tick) exp_tick[e] = st[e].t_out;
        if (exp_pkt_hops) exp_pkt_hops[e] = st[e].pkt_hops;
        if (exp_delivered) exp_delivered[e] = st[e].delivered;
        if (exp_digest) exp_digest[e] = st[e].digest;
        dead |= st[e].status == MSIM_EXP_DEADLOCK;
        inc |= st[e].status == MSIM_EXP_INCOMPLETE;
        fault |= st[e].status == MSIM_EXP_FAULT;
    }
    if (fault) return ctx_fail(ctx, MSIM_E_STATE, "an experiment reported an internal fault");
    return dead ? MSIM_S_DEADLOCK : (inc ? MSIM_S_INCOMPLETE : MSIM_OK);
}

extern "C" int msim_flow_count(const msim_ctx *ctx, uint32_t exp, uint64_t *n)
{
    if (!ctx || !n || exp >= ctx->n_exp) return MSIM_E_ARG;
    *n = ctx->exps[exp].n_flows;
    return MSIM_OK;
}

extern "C" int msim_flow_ticks(msim_ctx *ctx, uint32_t exp, void *stream, uint32_t *rd, uint32_t *act, uint32_t *sd)
{
    if (!ctx || exp >= ctx->n_exp) return MSIM_E_ARG;
    if (!ctx->bound) return ctx_fail(ctx, MSIM_E_STATE, "msim_flow_ticks before msim_bind");
    if (!ctx->recorded[exp]) return ctx_fail(ctx, MSIM_E_ARG, "experiment not recorded");
    hipError_t he = hipStreamSynchronize((hipStream_t)stream);
    const uint64_t n = ctx->exps[exp].n_flows;
    uint32_t *dst[3] = {rd, act, sd};
    for (int k = 0; k < 3 && he == hipSuccess; k++)
        if (dst[k] && n) he = hipMemcpy(dst[k], ctx->ws + ctx->rec_off[exp] + 4ull * k * n, 4ull * n, hipMemcpyDeviceToHost);
    if (he != hipSuccess) return hip_fail(ctx, he, "flow ticks copy");
    return MSIM_OK;
}

extern "C" int msim_task_count(const msim_ctx *ctx, uint32_t exp, uint32_t *n_tasks)
{
    if (!ctx || !n_tasks || exp >= ctx->n_exp) return MSIM_E_ARG;
    *n_tasks = ctx->exps[exp].n_task;
    return MSIM_OK;
}

extern "C" int msim_task_ticks(msim_ctx *ctx, uint32_t exp, void *stream, uint32_t *start, uint32_t *finish)
{
    if (!ctx || exp >= ctx->n_exp) return MSIM_E_ARG;
    if (!ctx->bound) return ctx_fail(ctx, MSIM_E_STATE, "msim_task_ticks before msim_bind");
    const Compiled &c = ctx->exps[exp];
    if (!c.n_task) return MSIM_OK;
    hipError_t he = hipStreamSynchronize((hipStream_t)stream);
    std::vector<TaskRW> tw(c.n_task);
    if (he == hipSuccess)
        he = hipMemcpy(tw.data(), ctx->ws + ctx->arena_off[exp] + c.o_trw, sizeof(TaskRW) * c.n_task, hipMemcpyDeviceToHost);
    if (he != hipSuccess) return hip_fail(ctx, he, "task ticks copy");
    for (uint32_t k = 0; k < c.n_task; k++) {
        if (start) start[k] = tw[k].start;
        if (finish) finish[k] = tw[k].finish;
    }
    return MSIM_OK;
}

extern "C" int msim_get_info(const msim_ctx *ctx, msim_info *info)
{
    if (!ctx || !info) return MSIM_E_ARG;
    *info = ctx->info;
    return MSIM_OK;
}

extern "C" const char *msim_last_error(const msim_ctx *ctx)
{
    return ctx ? ctx->err.c_str() : g_create_error.c_str();
}

extern "C" void msim_destroy(msim_ctx *ctx) { delete ctx; }
