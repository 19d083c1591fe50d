/*
 * msim_kernel.hip -- persistent megakernel of the batched packet simulator
 * (gfx950 / CDNA4).
 *
 * One launch simulates a whole batch (Multiverse section 4.3: one kernel per
 * batch instead of one launch per system).  Unlike the pages' megakernel, which
 * moves every thread of the grid through one system at a time over all
 * experiments, each workgroup here claims one experiment at a time and runs its
 * whole tick loop alone: experiments never interact (single-process
 * multi-experiment, Multiverse section 2.2), so the only synchronisation is a
 * workgroup barrier between the phases of a tick.  The experiment's state
 * is copied into LDS when it fits; on the general path, when it does not, the
 * switch and NIC state, or else the port table, go to LDS and the rest is
 * worked on in place in HBM (each placement its own inlined copy of the tick
 * loop, so every access is an LDS or a global one).
 *
 * Tick t follows the step order of Multiverse section 3.2 (Schedule, Send,
 * NIC send, Forward, Transmit, NIC receive) with the forwarding pull-based as
 * in its section 4.2: every output pulls from the ingresses of its node.
 * Each kernel family folds that order into as few barrier-separated phases as
 * its data layout allows:
 *   general path (run_experiment): phase A, one thread per port, takes the
 *     arrivals of tick t (switch ingresses append to their virtual output
 *     queues; hosts take deliveries and activate the flows they enable);
 *     barrier; phase D, rounds m < rate, every output grants the first
 *     eligible input going round from its pointer and stages the packet for
 *     t + delay; barrier;
 *   compact and ring paths (run_compact, run_ring): one thread per port with
 *     every port of a switch inside one wavefront, so the arrivals and the
 *     forwarding of a tick run in program order within the wavefront and one
 *     barrier ends the tick.
 * Writers.  Most state has one writer per phase.  The exceptions are LDS
 * atomics between the ports of one switch, inside one wavefront: on the
 * compact path an output hands the slot it popped back to its ingress (OR)
 * and counts the pop (add); on the ring path an output hands back the
 * slot and an emptied-queue bit (OR) into a word the ingress and the port
 * feeding it read next tick, and an ingress marks a queue non-empty in its
 * output's word (OR).  Several ports of a
 * switch may hit the same word in one instruction; OR and add do not depend on
 * the order they are applied in, so results are identical on every run.  The
 * other atomics: each workgroup claiming its next experiment; on the
 * general path, where the ports of a switch span wavefronts, an output
 * returning a popped slot to its ingress's free mask (OR), counting the pop
 * into the word of the output feeding that ingress and updating its own word
 * (add), the congestion-control queue lengths (add) and ACK-pending masks
 * (OR) and the task-graph counts (subtract); and the periodic completion
 * checks of the compact path (OR, max).
 */
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "msim_layout.h"

#define CHECK_EVERY 16u
/* The compact path checks every CHECK_EVERY ticks for the first CHECK_LONG
 * ticks of a run, then every CHECK_EVERY_LONG.  On the k=8 fat-tree batch a
 * check cost close to a tick; an experiment that runs past CHECK_LONG ticks
 * overshoots its end by fewer than CHECK_EVERY_LONG ticks in which nothing
 * happens, and its results do not depend on when the end is seen. */
#define CHECK_LONG 4096u
#define CHECK_EVERY_LONG 256u
#define LDSP __attribute__((address_space(3)))

__device__ __forceinline__ uint64_t mix64(uint64_t z)
{
    /* SplitMix64 output function (Steele, Lea, Flood 2014; Vigna's constants) */
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

struct Ctx {
    const PortRO *port;
    const ConnRO *conn;
    const Grp *grp;
    const uint32_t *hout;
    const HostRO *host;
    uint8_t *tail, *nslot;
    uint32_t *pdesc;
    uint8_t *pnxt;
    uint64_t *fmask;
    uint32_t *ow, *qlen;
    uint8_t *hpc;        /* per host: connections whose flow finished sending last tick */
    PortRW *ps;
    uint8_t *scnt;
    uint32_t *sdesc;
    ConnRW *cs;
    HostRW *hs;
    uint32_t *ready;
    uint32_t n_ports, Q, W, R;
    uint32_t *rec;       /* per-flow ticks (rd | act | sd), or null */
    uint32_t n_flows;
    uint32_t n_task;     /* task graph */
    const TaskRO *task;
    const uint32_t *tpred;
    TaskRW *trw;
    uint32_t cc, ecn_k, WA, n_rdy;  /* congestion control */
    CcRW *ccs;
    QcnRW *qcs;         /* the same slots, DCQCN's view */
    HpRW *hps;          /* and HPCC's */
    uint32_t cshift, hx;/* descriptor: conn << cshift; HPCC: switches per telemetry record */
    uint32_t *hl, *hint;/* HPCC: last ACK's telemetry, telemetry records */
    uint16_t *ack;
    uint32_t *bl, *ackm;
    uint32_t sp, sbits, seed, n_hosts;   /* packet spraying */
    const uint32_t *spi, *rwoff;
    const uint16_t *cand;
    uint32_t *sseq, *rnext, *rbits;
};

/* 0x80 in every byte of d that is not zero */
__device__ __forceinline__ uint64_t bytes_nz(uint64_t d)
{
    const uint64_t L = 0x7F7F7F7F7F7F7F7Full;
    return ((((d & L) + L) | d) & ~L);
}

/* First set byte-flag at or after byte rr, cyclically over the row; -1 if none. */
template <int W>
__device__ __forceinline__ int first_from(uint64_t n0, uint64_t n1, uint32_t rr)
{
    if (W == 1) {
        const uint32_t sh = 8 * rr;
        uint64_t rot = sh ? (n0 >> sh) | (n0 << (64 - sh)) : n0;
        if (!rot) return -1;
        return (int)((rr + (__builtin_ctzll(rot) >> 3)) & 7);
    }
    uint64_t a = rr < 8 ? n0 : n1, b = rr < 8 ? n1 : n0;
    const uint32_t sh = 8 * (rr & 7), base = rr < 8 ? 0 : 8, other = 8 - base;
    uint64_t m = a & (~0ull << sh);
    if (m) return (int)(base + (__builtin_ctzll(m) >> 3));
    if (b) return (int)(other + (__builtin_ctzll(b) >> 3));
    m = a & ((1ull << sh) - 1ull);
    if (m) return (int)(base + (__builtin_ctzll(m) >> 3));
    return -1;
}

/* The first n (<= 16) bytes at p as two packed words, byte i at bits 8i..8i+7;
 * the loads are independent, so their latencies overlap. */
__device__ __forceinline__ void row_bytes(const uint8_t *p, uint32_t n, uint64_t &w0, uint64_t &w1)
{
    const uintptr_t ad = (uintptr_t)p;
    if (n == 16 && (ad & 15u) == 0) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = *(const u32x4 *)p;
        w0 = (uint64_t)v.x | ((uint64_t)v.y << 32);
        w1 = (uint64_t)v.z | ((uint64_t)v.w << 32);
        return;
    }
    if (n == 8 && (ad & 7u) == 0) {
        w0 = *(const uint64_t *)p;
        w1 = 0;
        return;
    }
    w0 = w1 = 0;
#pragma unroll
    for (uint32_t i = 0; i < 16; i++)
        if (i < n) {
            const uint64_t b = p[i];
            if (i < 8) w0 |= b << (8 * i);
            else w1 |= b << (8 * (i - 8));
        }
}

/* Byte o of a row held as two packed words, and its replacement. */
__device__ __forceinline__ uint32_t row_get(uint64_t w0, uint64_t w1, uint32_t o)
{
    return (uint32_t)(((o < 8 ? w0 : w1) >> (8 * (o & 7))) & 0xFFu);
}

__device__ __forceinline__ void row_set(uint64_t &w0, uint64_t &w1, uint32_t o, uint32_t v)
{
    const uint32_t sh = 8 * (o & 7);
    const uint64_t keep = ~(0xFFull << sh), b = (uint64_t)(v & 0xFFu) << sh;
    if (o < 8) w0 = (w0 & keep) | b;
    else w1 = (w1 & keep) | b;
}

struct Acc {
    uint64_t hops, delivered, digest;
    uint32_t tmax, last_tx1, last_act1, max_arr;
    uint32_t left;
    uint32_t fault;      /* set if an invariant the credits guarantee is ever broken */
};

/* ---------------------------------------------------------- flow schedule */

/* Chunk rank i sends at step s of a ring round (NCCL ring order). */
__device__ __forceinline__ uint32_t ring_chunk(uint32_t kind, uint32_t N, uint32_t i, uint32_t s)
{
    if (kind == GK_RING_AG || s < N - 1) return (i + N - s) % N;
    uint32_t s2 = s - (N - 1);
    return (i + 1 + N - s2) % N;
}

__device__ __forceinline__ uint32_t flows_per_conn(const Grp &g)
{
    switch (g.kind) {
    case GK_BCAST: return g.S;
    case GK_XFLOW:
    case GK_SEQ: return 1u;
    case GK_TREE: return g.R;
    default: return g.R * g.S;
    }
}

__device__ __forceinline__ uint32_t flow_size(const Grp &g, const ConnRO &cr, uint32_t pos)
{
    if (g.kind == GK_XFLOW) return cr.idx;
    if (g.kind == GK_SEQ) return g.p;
    if (g.kind == GK_TREE) return pos + 1 < g.R ? g.p : g.X;
    if (g.kind == GK_BCAST) return g.p / g.S + (pos < g.p % g.S ? 1u : 0u);
    uint32_t r = pos / g.S;
    if (r + 1 < g.R) return g.p;
    uint32_t s = pos - r * g.S;
    uint32_t k = ring_chunk(g.kind, g.N, cr.idx, s);
    return g.X / g.N + (k < g.X % g.N ? 1u : 0u);
}

__device__ __forceinline__ uint32_t flow_id(const Grp &g, const ConnRO &cr, uint32_t c, uint32_t pos)
{
    if (g.kind == GK_XFLOW) return g.fid_base + (c - g.conn_base);
    if (g.kind == GK_SEQ) return g.fid_base + cr.idx;
    if (g.kind == GK_TREE) return g.fid_base + pos * 2u * (g.N - 1u) + cr.idx;
    if (g.kind == GK_BCAST) return g.fid_base + cr.idx * g.S + pos;
    return g.fid_base + pos * g.N + cr.idx;
}

/* Tree connection j (up of member j+1 for j < N-1, else down of member
 * j-N+2): has chunk pos arrived from everything it waits on?  Up: from the
 * member's children; down from the root: from the root's children; other
 * down: at its source from above.  Connection of the up link of member i:
 * i-1; of its down link: N-1+i-1. */
template <typename RPos>
__device__ __forceinline__ bool tree_ready(uint32_t N, uint32_t j, uint32_t pos, RPos rpos)
{
    uint32_t ch;
    if (j < N - 1) {
        ch = 2 * (j + 1) + 1;                      /* first child of member j+1 */
    } else {
        const uint32_t i = j - (N - 1) + 1, par = (i - 1) / 2;
        if (par != 0) return rpos(N - 1 + par - 1) > pos;
        ch = 1;                                    /* the root's children */
    }
    if (ch < N && rpos(ch - 1) <= pos) return false;
    if (ch + 1 < N && rpos(ch) <= pos) return false;
    return true;
}

/* Tree connections whose next flow may wait on a flow just received over
 * connection j; calls f(index within the group) for each. */
template <typename F>
__device__ __forceinline__ void tree_dependents(uint32_t N, uint32_t j, F f)
{
    if (j < N - 1) {
        const uint32_t par = j / 2;                /* parent of member j+1 */
        if (par != 0) {
            f(par - 1);
        } else {
            f(N - 1);
            if (N > 2) f(N);
        }
    } else {
        const uint32_t i = j - (N - 1) + 1;
        for (uint32_t ch = 2 * i + 1; ch <= 2 * i + 2 && ch < N; ch++) f(N - 1 + ch - 1);
    }
}

/* Is the receive predecessor of flow `pos` of connection c met? (the ring's data
 * dependency on the previous step of rank i-1; the broadcast's dependency on the
 * same partition one hop earlier) */
__device__ __forceinline__ bool recv_ok(const Ctx &C, const Grp &g, const ConnRO &cr, uint32_t c,
                                        uint32_t pos)
{
    /* a collective a task names starts with the task: the first flow of each
     * of its connections waits for the task's start */
    if (pos == 0 && g.task != MSIM_NONE && C.trw[g.task].start == MSIM_NONE) return false;
    if (g.kind == GK_RING_AR || g.kind == GK_RING_AG) {
        uint32_t s = pos % g.S;
        if (s == 0) {
            /* a gated ring's first step waits for this rank's piece of the send/recv */
            if (pos == 0 && g.link != MSIM_NONE) return C.cs[C.grp[g.link].conn_base + cr.idx].r_pos >= 1;
            return true;
        }
        uint32_t cin = g.conn_base + (cr.idx + g.N - 1) % g.N;
        return C.cs[cin].r_pos >= pos;
    }
    if (g.kind == GK_BCAST) {
        if (cr.idx == 0) return true;
        return C.cs[c - 1].r_pos > pos;
    }
    if (g.kind == GK_SEQ) return cr.idx == 0 || (C.cs[c - 1].s_pos & CS_POS_MASK) >= 1;
    if (g.kind == GK_TREE)
        return tree_ready(g.N, cr.idx, pos, [&](uint32_t j) { return C.cs[g.conn_base + j].r_pos; });
    return true;
}

/* DCTCP (Alizadeh et al., SIGCOMM 2010) in integer arithmetic: may the
 * connection put another packet in flight? */
__device__ __forceinline__ bool window_open(const CcRW &q)
{
    return q.sent - q.acked < (q.cwnd >> 8);
}

/* k ACKs, m of them ECN-marked, reach the connection's source in one tick:
 * additive increase of 1/cwnd per unmarked ACK; at the end of each window of
 * data, alpha moves 1/16 of the way to the window's marked fraction and a
 * window that saw a mark shrinks by alpha/2. */
__device__ __forceinline__ void dctcp_acks(CcRW &q, uint32_t k, uint32_t m)
{
    q.acked += k;
    q.wa += k;
    q.wm += m;
    if (k > m) q.cwnd = (uint32_t)min((uint64_t)q.cwnd + (uint64_t)(k - m) * 65536u / q.cwnd, (uint64_t)CWND_MAX_FP);
    if (q.acked >= q.wend) {
        const uint32_t F = (uint32_t)((uint64_t)q.wm * 1024u / q.wa);
        q.alpha = q.alpha - (q.alpha >> 4) + (F >> 4);
        if (q.wm) {
            const uint32_t cut = (uint32_t)(((uint64_t)q.cwnd * q.alpha) >> 11);
            q.cwnd = max(q.cwnd - cut, 256u);
        }
        q.wend = q.sent;
        q.wa = q.wm = 0;
    }
}

/* DCQCN (Zhu et al., SIGCOMM 2015, section 3) at the source, in integer
 * arithmetic.  An increase event: the timer or byte-counter stage has just
 * grown.  Below F stages in both it is fast recovery (RT kept), beyond F in
 * both a hyper increase, else an additive one; RC then moves halfway to RT. */
__device__ __forceinline__ void qcn_increase(QcnRW &q)
{
    const uint32_t hi = max(q.tcnt, q.bcnt), lo = min(q.tcnt, q.bcnt);
    if (hi >= QCN_F) q.rt = min(q.rt + (lo > QCN_F ? (lo - QCN_F) * QCN_HAI : QCN_AI), QCN_ONE);
    q.rc = (q.rt + q.rc) >> 1;
}

/* Applies the timer events due by tick t in time order (alpha's decay before
 * the rate increase when both fall on one tick). */
__device__ __forceinline__ void qcn_timers(QcnRW &q, uint32_t t)
{
    uint32_t ni = q.next_inc, na = q.next_alpha;
    while (min(ni, na) <= t) {
        const uint32_t e = min(ni, na);
        if (na == e) { q.alpha -= q.alpha >> 8; na += QCN_PERIOD; }
        if (ni == e) { q.tcnt++; qcn_increase(q); ni += QCN_PERIOD; }
    }
    q.next_inc = ni;
    q.next_alpha = na;
}

/* A CNP reaches the source at t: the rate cut by alpha/2, alpha raised,
 * stages and timers restarted. */
__device__ __forceinline__ void qcn_cnp(QcnRW &q, uint32_t t)
{
    qcn_timers(q, t);
    q.rt = q.rc;
    q.rc = max(q.rc - (uint32_t)(((uint64_t)q.rc * q.alpha) >> 11), QCN_RMIN);
    q.alpha = q.alpha - (q.alpha >> 8) + 4u;
    q.tcnt = q.bcnt = q.bsent = 0;
    q.next_inc = q.next_alpha = t + QCN_PERIOD;
}

/* The source sent a packet at t: timers, byte counter, and the pacer's next
 * send time (which may lag the schedule by under one tick, so fractional gaps
 * average out).  Returns the first tick the connection may send again. */
__device__ __forceinline__ uint32_t qcn_sent(QcnRW &q, uint32_t t)
{
    qcn_timers(q, t);
    if (++q.bsent == QCN_BYTES) { q.bsent = 0; q.bcnt++; qcn_increase(q); }
    const uint64_t now = (uint64_t)t << 16, lag = now > 65535u ? now - 65535u : 0;
    q.next_fp = max(q.next_fp, lag) + (1ull << 32) / q.rc;
    return (uint32_t)((q.next_fp + 65535u) >> 16);
}

/* HPCC (Li et al., SIGCOMM 2019, Algorithm 1) at the source, in integer
 * arithmetic: may the connection put another packet in flight? */
__device__ __forceinline__ bool hp_open(const HpRW &h)
{
    return h.sent - h.acked < (h.w >> 8);
}

/* One ACK (acked already counted up for it) with the telemetry `rec` of the
 * packet it acknowledges, 3 words per switch; L holds the previous ACK's.
 * The utilisation sample of each switch with time between its two records,
 * the largest one folded into U, then the window; Wc and the stage move once
 * per round trip. */
__device__ __forceinline__ void hpcc_ack(HpRW &h, uint32_t *L, const uint32_t *rec)
{
    if (h.have) {
        const bool update = h.acked > h.hlast;
        const uint64_t T = h.T;
        uint64_t u = 0;
        uint32_t tau = 0;
        for (uint32_t i = 0; i < h.nsw; i++) {
            const uint32_t dts = rec[3 * i] - L[3 * i];
            if (dts == 0) continue;
            const uint32_t qb = rec[3 * i + 2];
            const uint64_t mq = min(qb & 0xFFFFFFu, L[3 * i + 2] & 0xFFFFFFu);
            const uint64_t up = (65536ull * (mq * dts + (uint64_t)(rec[3 * i + 1] - L[3 * i + 1]) * T)) /
                                ((uint64_t)(qb >> 24) * T * dts);
            if (up > u) { u = up; tau = dts; }
        }
        tau = (uint32_t)min((uint64_t)tau, T);
        h.U = (uint32_t)(((T - tau) * h.U + tau * u) / T);
        const uint64_t cap = T << 8;
        const bool mult = h.U >= HP_ETA || h.stage >= HP_MAX_STAGE;
        uint64_t w = mult ? (h.U ? (uint64_t)h.wc * HP_ETA / h.U : cap) + h.wai : (uint64_t)h.wc + h.wai;
        h.w = (uint32_t)max(min(w, cap), (uint64_t)256);
        if (update) {
            h.stage = mult ? 0 : h.stage + 1;
            h.wc = h.w;
            h.hlast = h.sent;
        }
    } else {
        h.have = 1;
        h.hlast = h.sent;
    }
    for (uint32_t i = 0; i < 3 * h.nsw; i++) L[i] = rec[i];
}

__device__ __forceinline__ void activate(const Ctx &C, Acc &a, uint32_t c, uint32_t pos, const Grp &g,
                                         const ConnRO &cr, uint32_t rdy_off, uint32_t t)
{
    C.cs[c].s_pos = pos | (CS_ACTIVE << CS_SHIFT);
    C.cs[c].s_rem = flow_size(g, cr, pos);
    /* with congestion control a closed window keeps it out of the NIC's
     * candidates until an ACK reopens it */
    const bool open = C.cc == CC_DCTCP ? window_open(C.ccs[c]) : C.cc == CC_HPCC ? hp_open(C.hps[c]) : true;
    if (open) C.ready[rdy_off + (cr.lidx >> 5)] |= 1u << (cr.lidx & 31);
    a.last_act1 = t + 1;
    if (C.rec) C.rec[C.n_flows + flow_id(g, cr, c, pos)] = t;
}

/* Activates connection d's next flow if it was waiting and is now ready.
 * Every caller passes a connection whose source is the calling host. */
__device__ __forceinline__ void wake(const Ctx &C, Acc &a, uint32_t d, uint32_t rdy_off, uint32_t t)
{
    if ((C.cs[d].s_pos >> CS_SHIFT) != CS_IDLE) return;
    const ConnRO dr = C.conn[d];
    const Grp dg = C.grp[dr.grp];
    const uint32_t dpos = C.cs[d].s_pos & CS_POS_MASK;
    if (recv_ok(C, dg, dr, d, dpos)) activate(C, a, d, dpos, dg, dr, rdy_off, t);
}

/* After a flow over connection c (group g) has been fully received: the
 * connections leaving this host whose next flow waits on it. */
__device__ __forceinline__ void wake_dependents(const Ctx &C, Acc &a, const Grp &g, const ConnRO &cr, uint32_t c,
                                                uint32_t rdy_off, uint32_t t)
{
    if (g.kind == GK_RING_AR || g.kind == GK_RING_AG) {
        wake(C, a, g.conn_base + (cr.idx + 1) % g.N, rdy_off, t);
    } else if (g.kind == GK_BCAST) {
        if (cr.idx + 1 < g.N) wake(C, a, c + 1, rdy_off, t);
    } else if (g.kind == GK_SEQ) {
        for (uint32_t k = 0; k < g.X; k++) wake(C, a, C.grp[g.link + k].conn_base + cr.idx, rdy_off, t);
    } else if (g.kind == GK_TREE) {
        tree_dependents(g.N, cr.idx, [&](uint32_t j) { wake(C, a, g.conn_base + j, rdy_off, t); });
    }
}

/* Phase-B decision for a connection whose previous flow has left (or at t = 0). */
__device__ __forceinline__ void check_conn(const Ctx &C, Acc &a, uint32_t c, uint32_t rdy_off, uint32_t t)
{
    const ConnRO cr = C.conn[c];
    const Grp g = C.grp[cr.grp];
    uint32_t pos = C.cs[c].s_pos & CS_POS_MASK;
    if (pos >= flows_per_conn(g)) {
        C.cs[c].s_pos = pos | (CS_DONE << CS_SHIFT);
        /* a send/recv's next receiver waits on this send (its SEND predecessor) */
        if (g.kind == GK_SEQ && cr.idx + 1 < g.N) wake(C, a, c + 1, rdy_off, t);
    } else if (recv_ok(C, g, cr, c, pos)) {
        activate(C, a, c, pos, g, cr, rdy_off, t);
    } else {
        C.cs[c].s_pos = pos | (CS_IDLE << CS_SHIFT);
    }
}

/* MurmurHash3's 32-bit finaliser (Appleby, public domain). */
__device__ __forceinline__ uint32_t fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

/* Packet spraying: the egress local port of packet (connection c, sequence
 * number seq) at switch `node` among the set bits of mask (the equal-cost
 * egresses, in port order); 0xFF if there is none. */
__device__ __forceinline__ uint32_t spray_pick(uint32_t mask, uint32_t c, uint32_t seq, uint32_t node, uint32_t seed)
{
    const uint32_t n = __builtin_popcount(mask);
    if (!n) return 0xFFu;
    const uint32_t key = c ^ fmix32(seq + 1u);
    uint32_t k = fmix32(key ^ fmix32(node ^ seed)) % n;
    for (; k; k--) mask &= mask - 1u;
    return (uint32_t)__builtin_ctz(mask);
}

/* ---------------------------------------------------------------- phase A */

__device__ __forceinline__ void phase_a_host(const Ctx &C, Acc &a, uint32_t p, const PortRO &pr,
                                             uint32_t t, uint32_t slot)
{
    const uint32_t si = p * C.W + slot;
    const uint32_t n = C.scnt[si];
    /* without congestion control a host has nothing to do in a tick with no
     * arrival and no flow that finished sending in the last one */
    const uint32_t np = C.hpc[pr.host];
    if (!C.cc && n == 0 && np == 0 && t != 0) return;
    const HostRO hr = C.host[pr.host];
    HostRW &hw = C.hs[pr.host];
    if (C.cc) {
        /* the ACKs due now at this host's outgoing connections: the pending
         * masks name the connections that have some */
        const uint32_t as = t & (C.WA - 1);
        uint32_t *pend = C.ackm + as * C.n_rdy + hr.rdy_off;
        for (uint32_t w = 0; w < (hr.n_out + 31) / 32; w++) {
            uint32_t m = pend[w];
            if (!m) continue;
            pend[w] = 0;
            for (; m; m &= m - 1) {
            const uint32_t j = 32 * w + __builtin_ctz(m);
            const uint32_t c = C.hout[hr.out_off + j];
            const uint32_t v = C.ack[c * C.WA + as];
            C.ack[c * C.WA + as] = 0;
            if (C.cc == CC_DCQCN) {
                qcn_cnp(C.qcs[c], t);     /* at most one: CNPs are 608 ticks apart */
                continue;
            }
            bool open;
            if (C.cc == CC_HPCC) {
                /* ACKs one by one, in sequence order, each with its packet's
                 * telemetry record */
                HpRW &h = C.hps[c];
                uint32_t *L = C.hl + 3 * C.hx * c;
                for (uint32_t i = v & 0xFFu; i; i--) {
                    const uint32_t seq = h.acked++;
                    hpcc_ack(h, L, C.hint + 3 * C.hx * (h.int_off + seq % h.slots));
                }
                open = hp_open(h);
            } else {
                CcRW &q = C.ccs[c];
                dctcp_acks(q, v & 0xFFu, v >> 8);
                open = window_open(q);
            }
            /* a grown window may let a waiting flow send again, and a window cut
             * below the packets in flight stops it */
            const uint32_t bit = 1u << (j & 31);
            if ((C.cs[c].s_pos >> CS_SHIFT) == CS_ACTIVE && C.cs[c].s_rem && open)
                C.ready[hr.rdy_off + (j >> 5)] |= bit;
            else
                C.ready[hr.rdy_off + (j >> 5)] &= ~bit;
            }
        }
    }
    for (uint32_t k = 0; k < n; k++) {
        const uint32_t desc = C.sdesc[si * C.R + k];
        uint32_t c, in_order = 1;
        if (C.sp) {
            /* sprayed: note the arrival, then hand over every packet of the
             * connection that is now in order (this one may hold back none,
             * or release several that overtook it) */
            c = desc >> C.sbits;
            const uint32_t seq = desc & ((1u << C.sbits) - 1u);
            uint32_t *bits = C.rbits + C.rwoff[c];
            bits[seq >> 5] |= 1u << (seq & 31);
            const uint32_t lim = (C.rwoff[c + 1] - C.rwoff[c]) * 32u;
            uint32_t r = C.rnext[c];
            in_order = 0;
            while (r < lim && ((bits[r >> 5] >> (r & 31)) & 1u)) { r++; in_order++; }
            C.rnext[c] = r;
        } else {
            c = (desc & ~DESC_MARK) >> C.cshift;
        }
        ConnRW &cw = C.cs[c];
        a.delivered++;
        if (C.cc) {
            /* DCTCP: the packet's ACK; DCQCN: a CNP for a marked packet, at most
             * one per connection every 608 ticks.  It reaches the source one
             * path latency later; the source's pending mask for that tick gets
             * the connection's bit (other destinations may set bits of the same
             * word) */
            bool notify = true;
            if (C.cc == CC_DCQCN) {
                QcnRW &q = C.qcs[c];
                notify = (desc & DESC_MARK) && (q.last_cnp == MSIM_NONE || t - q.last_cnp >= QCN_CNP_GAP);
                if (notify) q.last_cnp = t;
            }
            if (notify) {
                const CcRW &q = C.ccs[c];
                const uint32_t ta = t + q.lat, as = ta & (C.WA - 1);
                C.ack[c * C.WA + as] += 1u + ((desc >> 31) << 8);
                atomicOr(C.ackm + as * C.n_rdy + q.aword, 1u << (C.conn[c].lidx & 31));
                a.max_arr = max(a.max_arr, ta);
            }
        }
        for (; in_order; in_order--) {
        if (--cw.r_rem != 0) continue;
        const ConnRO cr = C.conn[c];
        const Grp g = C.grp[cr.grp];
        uint32_t pos = cw.r_pos;
        uint32_t fid = flow_id(g, cr, c, pos);
        a.digest += mix64(((uint64_t)fid << 32) | t);
        a.tmax = max(a.tmax, t);         /* a task this lane started may finish later */
        a.left--;
        hw.left--;
        if (C.rec) C.rec[fid] = t;
        pos++;
        cw.r_pos = pos;
        if (pos < flows_per_conn(g)) cw.r_rem = flow_size(g, cr, pos);
        /* the last flow of a collective task's collective finishes the task
         * (hosts count down concurrently) */
        if (g.task != MSIM_NONE && atomicSub(&C.trw[g.task].left, 1u) == 1u) C.trw[g.task].finish = t;
        wake_dependents(C, a, g, cr, c, hr.rdy_off, t);
        }
    }
    if (n) C.scnt[si] = 0;
    /* activations (phase B of the tick) */
    if (t == 0) {
        for (uint32_t j = 0; j < hr.n_out; j++) check_conn(C, a, C.hout[hr.out_off + j], hr.rdy_off, t);
    } else {
        for (uint32_t k = 0; k < np; k++) check_conn(C, a, hw.pend[k], hr.rdy_off, t);
        if (np) C.hpc[pr.host] = 0;
    }
}

/* Schedule (tasks k = first, first + stride, ...): a task starts at the first
 * tick by which all its predecessors have finished; a compute or intra-server
 * task's finish is then known.  Durations are >= 1 tick, so a task started
 * now cannot let another one start in the same tick.  Returns whether one
 * started. */
__device__ __forceinline__ bool schedule_tasks(const Ctx &C, Acc &a, uint32_t first, uint32_t stride, uint32_t t)
{
    bool started = false;
    for (uint32_t k = first; k < C.n_task; k += stride) {
        TaskRW &tw = C.trw[k];
        if (tw.start != MSIM_NONE) continue;
        const TaskRO tk = C.task[k];
        bool ok = true;
        for (uint32_t q = 0; q < tk.npred && ok; q++) {
            const uint32_t fin = C.trw[C.tpred[tk.pred_off + q]].finish;
            ok = fin != MSIM_NONE && fin <= t;
        }
        if (!ok) continue;
        tw.start = t;
        started = true;
        a.last_act1 = t + 1;
        if (tk.type != TK_COLL) {
            tw.finish = t + tk.dur;
            a.max_arr = max(a.max_arr, tw.finish);
            a.tmax = max(a.tmax, tw.finish);
        }
    }
    return started;
}

/* A host's connections whose collective's task started this tick. */
__device__ __forceinline__ void task_wake_host(const Ctx &C, Acc &a, const PortRO &pr, uint32_t t)
{
    const HostRO hr = C.host[pr.host];
    for (uint32_t j = 0; j < hr.n_out; j++) {
        const uint32_t c = C.hout[hr.out_off + j];
        const uint32_t tk = C.grp[C.conn[c].grp].task;
        if (tk != MSIM_NONE && C.trw[tk].start == t) wake(C, a, c, hr.rdy_off, t);
    }
}

/* Has every task finished by tick t - 1? (threads k = first, first + stride, ...) */
__device__ __forceinline__ bool tasks_pending(const Ctx &C, uint32_t first, uint32_t stride, uint32_t t)
{
    for (uint32_t k = first; k < C.n_task; k += stride) {
        const TaskRW tw = C.trw[k];
        if (tw.start == MSIM_NONE || tw.finish == MSIM_NONE || tw.finish >= t) return true;
    }
    return false;
}

__device__ __forceinline__ void phase_a_switch(const Ctx &C, Acc &a, uint32_t q, const PortRO &pr, uint32_t slot)
{
    /* the packets that arrive now, if any, join the queue toward the egress
     * their route names; nothing else happens at an ingress */
    const uint32_t si = q * C.W + slot;
    const uint32_t n = C.scnt[si];
    if (n == 0) return;
    const uint32_t deg = pr.deg, i = pr.local, Q = C.Q;
    const uint32_t qp = pr.host + i;               /* this ingress's buffer pool */
    /* its free slots: a 256-bit mask the outputs return slots to */
    uint64_t *fm = C.fmask + 4u * qp;
    const uint32_t nw = (Q + 63u) >> 6;
    uint64_t m0 = fm[0], m1 = nw > 1 ? fm[1] : 0ull, m2 = nw > 2 ? fm[2] : 0ull, m3 = nw > 3 ? fm[3] : 0ull;
    for (uint32_t k = 0; k < n; k++) {
        uint32_t desc = C.sdesc[si * C.R + k];
        uint32_t c, o;
        if (C.sp) {
            /* sprayed: this switch's equal-cost egresses toward the destination,
             * in the climbing state the ingress implies, picked by the hash */
            c = desc >> C.sbits;
            const uint32_t info = C.spi[q];
            const uint32_t row = (info >> 16) & 0x7FFFu;
            const uint32_t mask = C.cand[((size_t)row * C.n_hosts + C.conn[c].route) * 2u + (info >> 31)];
            o = spray_pick(mask, c, desc & ((1u << C.sbits) - 1u), info & 0xFFFFu, C.seed);
        } else {
            c = (desc & ~DESC_MARK) >> C.cshift;
            o = (C.conn[c].route >> (4 * (desc & DESC_HOP_MASK))) & 0xFu;
        }
        /* the lowest free slot */
        uint32_t s;
        if (m0) { s = (uint32_t)__builtin_ctzll(m0); m0 &= m0 - 1; }
        else if (m1) { s = 64u + (uint32_t)__builtin_ctzll(m1); m1 &= m1 - 1; }
        else if (m2) { s = 128u + (uint32_t)__builtin_ctzll(m2); m2 &= m2 - 1; }
        else if (m3) { s = 192u + (uint32_t)__builtin_ctzll(m3); m3 &= m3 - 1; }
        else s = Q_EMPTY;
        if (s == Q_EMPTY || o >= deg) { a.fault = 1; continue; }   /* cannot happen while credits hold */
        /* ECN: marked when the egress's backlog before this tick reaches K */
        if (C.cc && C.bl[pr.base + o] >= C.ecn_k) desc |= DESC_MARK;
        C.pdesc[qp * Q + s] = C.sp ? desc : desc + 1;    /* ECMP: on to the next switch of the route */
        /* an empty queue (head byte Q_EMPTY) gets s as its head, else s goes
         * behind its tail */
        const uint32_t vp = pr.vbase + o * deg + i;
        if (C.nslot[vp] == Q_EMPTY) C.nslot[vp] = (uint8_t)s;
        else C.pnxt[qp * Q + C.tail[vp]] = (uint8_t)s;
        C.tail[vp] = (uint8_t)s;
        if (C.cc) __hip_atomic_fetch_add(C.qlen + pr.base + o, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    C.scnt[si] = 0;
    fm[0] = m0;
    if (nw > 1) fm[1] = m1;
    if (nw > 2) fm[2] = m2;
    if (nw > 3) fm[3] = m3;
}

/* ---------------------------------------------------------------- phase D */

/* The m-th packet an output sends in tick t.  Only this output stages packets
 * at its far ingress, and that ingress empties the slot of arrival tick t + d
 * when it reads it, W > d ticks before this output uses the slot again; so the
 * slot holds exactly the m packets sent before this one in this tick. */
__device__ __forceinline__ void transmit(const Ctx &C, Acc &a, uint32_t p, const PortRO &pr, uint32_t desc,
                                         uint32_t t, uint32_t m)
{
    uint32_t ta = t + pr.delay;
    uint32_t si = pr.peer * C.W + ta % C.W;
    C.scnt[si] = (uint8_t)(m + 1);
    C.sdesc[si * C.R + m] = desc;
    a.hops++;
    a.last_tx1 = t + 1;
    a.max_arr = max(a.max_arr, ta);
}

/* Output p's word: packets sent and not yet forwarded by the far ingress
 * (bits 0-7), the packets the far switch's outputs took from that ingress
 * during ticks of parity 0 (bits 8-15) and 1 (bits 16-23), and a switch
 * output's round-robin pointer (bits 24-31).  Those outputs add to the byte
 * of their tick's parity; p, at tick t, reads the byte of t - 1, takes it off
 * its in-flight count and clears it with one atomic add that also records
 * what it sent, so neither side overwrites the other's byte. */
__device__ __forceinline__ uint32_t pops_shift(uint32_t t) { return 8u + 8u * (t & 1u); }

__device__ __forceinline__ void phase_d_host(const Ctx &C, Acc &a, uint32_t p, const PortRO &pr, uint32_t t)
{
    const HostRO hr = C.host[pr.host];
    if (!pr.alive || hr.n_out == 0) return;
    PortRW &pw = C.ps[p];
    const uint32_t ow = C.ow[p], shp = pops_shift(t + 1u);
    const uint32_t pp = (ow >> shp) & 0xFFu;
    int32_t credit = (int32_t)C.Q - (int32_t)((ow & 0xFFu) - pp);
    uint32_t rr = pw.rr, pushed = 0;
    const uint32_t nw = (hr.n_out + 31) >> 5;
    uint32_t *rdy = C.ready + hr.rdy_off;
    HostRW &hw = C.hs[pr.host];
    bool moved = false;
    for (uint32_t m = 0; m < pr.rate && credit > 0; m++) {
        /* first ready connection at or after rr, cyclically */
        uint32_t w0 = rr >> 5, b0 = rr & 31, j = MSIM_NONE;
        for (uint32_t k = 0; k <= nw; k++) {
            uint32_t w = w0 + k;
            if (w >= nw) w -= nw;
            uint32_t bits = rdy[w];
            if (k == 0) bits &= ~0u << b0;
            else if (k == nw) bits &= (1u << b0) - 1u;
            if (C.cc == CC_DCQCN) {
                /* DCQCN: skip connections their pacer holds back */
                for (; bits; bits &= bits - 1) {
                    const uint32_t jj = (w << 5) + __builtin_ctz(bits);
                    if (((uint64_t)t << 16) >= C.qcs[C.hout[hr.out_off + jj]].next_fp) { j = jj; break; }
                }
                if (j != MSIM_NONE) break;
            } else if (bits) { j = (w << 5) + __builtin_ctz(bits); break; }
        }
        if (j == MSIM_NONE) break;
        uint32_t c = C.hout[hr.out_off + j];
        uint32_t desc = c << C.cshift;
        if (C.sp) desc = (c << C.sbits) | C.sseq[c]++;
        else if (C.cc == CC_HPCC) desc |= (C.hps[c].sent % C.hps[c].slots) << 4;   /* its telemetry record */
        transmit(C, a, p, pr, desc, t, m);
        pushed++;
        credit--;
        moved = true;
        rr = j + 1 == hr.n_out ? 0 : j + 1;
        ConnRW &cw = C.cs[c];
        if (C.cc == CC_DCTCP) {
            CcRW &q = C.ccs[c];
            q.sent++;
            if (!window_open(q)) rdy[j >> 5] &= ~(1u << (j & 31));
        } else if (C.cc == CC_DCQCN) {
            a.max_arr = max(a.max_arr, qcn_sent(C.qcs[c], t));
        } else if (C.cc == CC_HPCC) {
            HpRW &h = C.hps[c];
            h.sent++;
            if (!hp_open(h)) rdy[j >> 5] &= ~(1u << (j & 31));
        }
        if (--cw.s_rem == 0) {
            rdy[j >> 5] &= ~(1u << (j & 31));
            uint32_t pos = cw.s_pos & CS_POS_MASK;
            if (C.rec) {
                const ConnRO cr = C.conn[c];
                C.rec[2 * C.n_flows + flow_id(C.grp[cr.grp], cr, c, pos)] = t + 1;
            }
            cw.s_pos = (pos + 1) | (CS_WAIT << CS_SHIFT);
            hw.pend[C.hpc[pr.host]++] = c;
        }
    }
    if (moved) pw.rr = rr;
    const uint32_t delta = (pushed - pp) - (pp << shp);
    if (delta) __hip_atomic_fetch_add(C.ow + p, delta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void phase_d_switch(const Ctx &C, Acc &a, uint32_t p, const PortRO &pr, uint32_t t)
{
    if (!pr.alive) return;
    const uint32_t deg = pr.deg, lo = pr.local, Q = C.Q;
    PortRW &pw = C.ps[p];
    const uint32_t prow = pr.vbase + lo * deg;     /* popper-major row of this output */
    /* each input's queue toward this output: its head slot, Q_EMPTY when empty */
    uint64_t h0, h1;
    row_bytes(C.nslot + prow, deg, h0, h1);
    const uint32_t ow = C.ow[p], shp = pops_shift(t + 1u);
    const uint32_t pp = (ow >> shp) & 0xFFu;
    int32_t credit = pr.peer_is_host ? (int32_t)pr.rate : (int32_t)Q - (int32_t)((ow & 0xFFu) - pp);
    /* 0x80 in the byte of every input whose queue holds a packet */
    const uint64_t k0 = deg >= 8 ? ~0ull : (1ull << (8 * deg)) - 1ull;
    const uint64_t k1 = deg >= 16 ? ~0ull : deg <= 8 ? 0ull : (1ull << (8 * (deg - 8))) - 1ull;
    uint64_t e0 = bytes_nz(~h0) & k0, e1 = bytes_nz(~h1) & k1;
    const uint32_t rr0 = ow >> 24;
    uint32_t rr = rr0, pushed = C.cc == CC_HPCC ? pw.pushed : 0u;
    uint32_t taken = 0;
    for (uint32_t m = 0; m < pr.rate && credit > 0; m++) {
        const int jj = first_from<2>(e0, e1, rr);
        if (jj < 0) break;
        const uint32_t j = (uint32_t)jj;
        const uint32_t vp = prow + j;
        const uint32_t qi = pr.host + j;           /* switch ports: pr.host is the pool of port 0 */
        const uint32_t s = row_get(h0, h1, j);
        const uint32_t desc = C.pdesc[qi * Q + s];
        /* popping the tail empties the queue */
        const uint32_t nh = s == C.tail[vp] ? Q_EMPTY : C.pnxt[qi * Q + s];
        C.nslot[vp] = (uint8_t)nh;
        row_set(h0, h1, j, nh);
        if (nh == Q_EMPTY) {
            if (j < 8) e0 &= ~(0x80ull << (8 * j)); else e1 &= ~(0x80ull << (8 * (j - 8)));
        }
        /* the slot goes back to input j's free mask, and the pop into the
         * count the output feeding input j reads next tick */
        __hip_atomic_fetch_or(C.fmask + 4u * qi + (s >> 6), 1ull << (s & 63u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(C.ow + C.port[pr.base + j].peer, 1u << pops_shift(t), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        rr = j + 1 == deg ? 0 : j + 1;
        if (C.cc == CC_HPCC) {
            /* telemetry of this switch (the descriptor counts the switches
             * reached): tick, egress packets sent, backlog at the tick's
             * start | rate << 24 */
            const uint32_t c = desc >> C.cshift, slot = (desc >> 4) & ((1u << (C.cshift - 4)) - 1u);
            uint32_t *r = C.hint + 3 * (C.hx * (C.hps[c].int_off + slot) + (desc & DESC_HOP_MASK) - 1);
            r[0] = t;
            r[1] = pushed + 1;
            r[2] = C.bl[p] | (pr.rate << 24);
        }
        transmit(C, a, p, pr, desc, t, m);
        pushed++;
        credit--;
        taken++;
    }
    if (C.cc == CC_HPCC && taken) pw.pushed = pushed;
    /* an output toward a host counts nothing in flight */
    const uint32_t delta = (pr.peer_is_host ? 0u : taken - pp) - (pp << shp) + ((rr - rr0) << 24);
    if (delta) __hip_atomic_fetch_add(C.ow + p, delta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    /* packets arrived and not yet forwarded: what next tick's arrivals see */
    if (C.cc) {
        const uint32_t ql = C.qlen[p] - taken;
        C.qlen[p] = ql;
        C.bl[p] = ql;
    }
}

/* ------------------------------------------------------------ reductions */

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v)
{
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
        lo = (uint32_t)__shfl_xor((int)lo, o, 64);
        hi = (uint32_t)__shfl_xor((int)hi, o, 64);
        v += ((uint64_t)hi << 32) | lo;
    }
    return v;
}

struct Shared {
    uint32_t exp;
    uint32_t chk_any[2][16];
    uint32_t chk_max[2][16];
    uint32_t chk_net[2][16];   /* task graphs: the network's last busy tick, per wavefront */
    uint32_t chk_nxt[2][16];   /* ... and the next finish of a running task */
    uint64_t sum[3][16];
    uint32_t mx[5][16];
};

/* Folds the workgroup's totals of a run into the experiment's state (thread 0). */
__device__ void finish_state(ExpState *stp, const Shared &sh, uint32_t nwaves, uint32_t t, bool done, bool dead,
                             uint32_t t_dead)
{
    uint64_t h = 0, d = 0, g = 0;
    uint32_t tm = 0, lt = 0, la = 0, ma = 0, fa = 0;
    for (uint32_t w = 0; w < nwaves; w++) {
        h += sh.sum[0][w]; d += sh.sum[1][w]; g += sh.sum[2][w];
        tm = max(tm, sh.mx[0][w]); lt = max(lt, sh.mx[1][w]); la = max(la, sh.mx[2][w]); ma = max(ma, sh.mx[3][w]);
        fa = max(fa, sh.mx[4][w]);
    }
    ExpState st = *stp;
    st.pkt_hops += h;
    st.delivered += d;
    st.digest += g;
    st.t_max = max(st.t_max, tm);
    st.last_tx1 = max(st.last_tx1, lt);
    st.last_act1 = max(st.last_act1, la);
    st.max_arr = max(st.max_arr, ma);
    st.t_now = t;
    st.fault |= fa;
    if (st.fault) { st.status = 3; st.t_out = t; }
    else if (done) { st.status = 0; st.t_out = st.t_max; }
    else if (dead) { st.status = 2; st.t_out = t_dead; }
    else { st.status = 1; st.t_out = t; }
    *stp = st;
}

/* ----------------------------------------------------------- one experiment */

/* Where an experiment's arena lives while it runs.  A compile-time choice,
 * so that every array is addressed as LDS or as global memory, never
 * generically (a generic access's wait covers both LDS and memory). */
enum { PL_LDS = 0, PL_SPLIT = 1, PL_PORTS = 2, PL_HBM = 3 };

template <int PL, bool TASKS, bool CC, bool SP>
__device__ __attribute__((always_inline)) void run_experiment(const KParams &kp, uint32_t x, uint8_t *arena_g,
                                                              uint8_t *lds, Shared &sh)
{
    constexpr bool IN_LDS = PL == PL_LDS;
    const uint32_t tid = threadIdx.x, nth = blockDim.x;
    const uint32_t lane = tid & 63, wave = tid >> 6, nwaves = (nth + 63) >> 6;
    ExpState *stp = (ExpState *)(kp.ws + kp.o_state) + x;
    const ArenaHdr *H = (const ArenaHdr *)arena_g;
    const uint32_t arena_bytes = H->bytes, rw_off = H->rw_off;
    const uint32_t ro_hot = H->ro_hot, rw_hot = H->rw_hot;
    /* placement (chosen by place_of): the whole arena in LDS; else, if it
     * fits, only the switch / NIC state ([0, ro_hot) then [rw_off, rw_hot),
     * back to back); else, if it fits, only the port table, which every port
     * reads twice a tick; else all in HBM */
    constexpr bool split = PL == PL_SPLIT, ports = PL == PL_PORTS;
    const uint32_t port_b = (H->n_ports * (uint32_t)sizeof(PortRO) + 15u) & ~15u;
    if (ports) {
        const uint4 *src = (const uint4 *)(arena_g + H->o_port);
        uint4 *dst = (uint4 *)lds;
        for (uint32_t i = tid; i < port_b / 16; i += nth) dst[i] = src[i];
        __syncthreads();
    }
    if (IN_LDS || split) {
        const uint4 *src = (const uint4 *)arena_g;
        uint4 *dst = (uint4 *)lds;
        const uint32_t n0 = (IN_LDS ? arena_bytes : ro_hot) / 16;
        for (uint32_t i = tid; i < n0; i += nth) dst[i] = src[i];
        if (split) {
            const uint4 *s2 = (const uint4 *)(arena_g + rw_off);
            uint4 *d2 = (uint4 *)(lds + ro_hot);
            for (uint32_t i = tid; i < (rw_hot - rw_off) / 16; i += nth) d2[i] = s2[i];
        }
        __syncthreads();
    }
    /* The layout puts the switch and NIC state (port, host and sprayed-port
     * tables; queues, pools, staging, port and host state, backlogs, ACK
     * masks, ready words: the arrays taken with hot() below) in [0, ro_hot)
     * and [rw_off, rw_hot), and the per-connection and per-task state (taken
     * with cold()) outside them; the host checks that every array lies on its
     * side.  So each array's place is known here at compile time and
     * addressed as LDS or as global memory, never generically. */
    auto hot = [&](uint32_t off) -> uint8_t * {
        if constexpr (PL == PL_LDS) return lds + off;
        else if constexpr (PL == PL_SPLIT) return off < ro_hot ? lds + off : lds + ro_hot + (off - rw_off);
        else return arena_g + off;
    };
    auto cold = [&](uint32_t off) -> uint8_t * {
        if constexpr (PL == PL_LDS) return lds + off;
        else return arena_g + off;
    };
    Ctx C;
    C.port = ports ? (const PortRO *)lds : (const PortRO *)hot(H->o_port);
    C.conn = (const ConnRO *)cold(H->o_conn);
    C.grp = (const Grp *)cold(H->o_grp);
    C.hout = (const uint32_t *)cold(H->o_hout);
    C.host = (const HostRO *)hot(H->o_host);
    C.tail = hot(H->o_tail);
    C.nslot = hot(H->o_nslot);
    C.pdesc = (uint32_t *)hot(H->o_pdesc);
    C.pnxt = hot(H->o_pnxt);
    C.fmask = (uint64_t *)hot(H->o_fmask);
    C.ow = (uint32_t *)hot(H->o_ow);
    C.hpc = hot(H->o_hpc);
    C.qlen = (uint32_t *)hot(H->o_qlen);
    C.ps = (PortRW *)hot(H->o_pstate);
    C.scnt = hot(H->o_scnt);
    C.sdesc = (uint32_t *)hot(H->o_sdesc);
    C.cs = (ConnRW *)cold(H->o_cstate);
    C.hs = (HostRW *)hot(H->o_hstate);
    C.ready = (uint32_t *)hot(H->o_ready);
    C.n_ports = H->n_ports;
    C.Q = H->Q;
    C.W = H->W;
    C.R = H->R;
    C.n_flows = H->n_flows;
    C.n_task = H->n_task;
    C.task = (const TaskRO *)cold(H->o_task);
    C.tpred = (const uint32_t *)cold(H->o_tpred);
    C.trw = (TaskRW *)cold(H->o_trw);
    /* a compile-time 0 in the kernels without congestion control removes its
     * code (and registers) from them */
    C.cc = CC ? H->cc : 0u;
    C.ecn_k = H->ecn_k;
    C.WA = H->WA;
    C.ccs = (CcRW *)cold(H->o_cc);
    C.qcs = (QcnRW *)cold(H->o_cc);
    C.hps = (HpRW *)cold(H->o_cc);
    C.cshift = CC ? H->cshift : (uint32_t)DESC_SHIFT;
    C.hx = H->hx;
    C.hl = (uint32_t *)cold(H->o_hl);
    C.hint = (uint32_t *)cold(H->o_int);
    C.ack = (uint16_t *)cold(H->o_ack);
    C.bl = (uint32_t *)hot(H->o_bl);
    C.ackm = (uint32_t *)hot(H->o_ackm);
    C.n_rdy = H->n_rdy;
    C.sp = SP ? H->lb : 0u;       /* a compile-time 0 elsewhere, as for C.cc */
    C.sbits = H->sbits;
    C.seed = H->seed;
    C.n_hosts = H->n_hosts;
    C.spi = (const uint32_t *)hot(H->o_spi);
    C.cand = (const uint16_t *)cold(H->o_cand);
    C.rwoff = (const uint32_t *)cold(H->o_rwoff);
    C.sseq = (uint32_t *)cold(H->o_sseq);
    C.rnext = (uint32_t *)cold(H->o_rnext);
    C.rbits = (uint32_t *)cold(H->o_rbits);
    uint64_t roff = ((const uint64_t *)(kp.ws + kp.o_rec_off))[x];
    C.rec = roff == ~0ull ? nullptr : (uint32_t *)(kp.ws + roff);

    const uint32_t t0 = stp->t_now;
    const uint32_t t_end = (uint64_t)t0 + kp.max_ticks > 0xFFFFFFF0ull ? 0xFFFFFFF0u : t0 + kp.max_ticks;
    const uint32_t hist = max(max(stp->last_tx1, stp->last_act1), stp->max_arr);
    /* task graphs without congestion control or spraying (whose timers and
     * sequence numbers advance with the clock) may skip the ticks of an idle
     * network; hist_net: the network's last busy tick in earlier runs */
    constexpr bool SKIP = TASKS && !CC && !SP;
    const uint32_t hist_net = max(stp->last_tx1 ? stp->last_tx1 + C.W - 2u : 0u, stp->last_act1);

    Acc a;
    a.hops = a.delivered = a.digest = 0;
    a.tmax = a.last_tx1 = a.last_act1 = a.max_arr = 0;
    a.left = 0;
    a.fault = 0;
    for (uint32_t p = tid; p < C.n_ports; p += nth) {
        const PortRO &pr = C.port[p];
        if (pr.is_host) a.left += C.hs[pr.host].left;
    }

    uint32_t t = t0, par = 0, slot = t0 % C.W;
    bool done = false, dead = false;
    uint32_t t_dead = 0;
    while (t < t_end) {
        for (uint32_t p = tid; p < C.n_ports; p += nth) {
            const PortRO pr = C.port[p];
            if (pr.is_host) phase_a_host(C, a, p, pr, t, slot);
            else phase_a_switch(C, a, p, pr, slot);
        }
        __syncthreads();
        if (TASKS && C.n_task) {
            /* Schedule, then the first flows of collectives whose task started */
            if (__syncthreads_or(schedule_tasks(C, a, tid, nth, t))) {
                for (uint32_t p = tid; p < C.n_ports; p += nth) {
                    const PortRO pr = C.port[p];
                    if (pr.is_host) task_wake_host(C, a, pr, t);
                }
                __syncthreads();
            }
        }
        for (uint32_t p = tid; p < C.n_ports; p += nth) {
            const PortRO pr = C.port[p];
            if (pr.is_host) phase_d_host(C, a, p, pr, t);
            else phase_d_switch(C, a, p, pr, t);
        }
        t++;
        slot = slot + 1 == C.W ? 0 : slot + 1;
        if ((t - t0) % CHECK_EVERY == 0 || t == t_end) {
            uint32_t any = __ballot(a.left > 0 || (TASKS && tasks_pending(C, tid, nth, t))) != 0ull;
            uint32_t ts = wave_max_u32(max(max(a.last_tx1, a.last_act1), a.max_arr));
            if (lane == 0) { sh.chk_any[par][wave] = any; sh.chk_max[par][wave] = ts; }
            if constexpr (SKIP) {
                /* the network's last busy tick: the last arrival a transmission
                 * can make (delay < W) and the last activation; and the first
                 * tick at which a running task finishes */
                const uint32_t net = wave_max_u32(max(a.last_tx1 ? a.last_tx1 + C.W - 2u : 0u, a.last_act1));
                uint32_t nx = MSIM_NONE;
                for (uint32_t k = tid; k < C.n_task; k += nth) {
                    const TaskRW tw = C.trw[k];
                    if (tw.start != MSIM_NONE && tw.finish != MSIM_NONE && tw.finish >= t) nx = min(nx, tw.finish);
                }
                nx = wave_min_u32(nx);
                if (lane == 0) { sh.chk_net[par][wave] = net; sh.chk_nxt[par][wave] = nx; }
            }
            __syncthreads();
            any = 0;
            ts = hist;
            uint32_t net = hist_net, nx = MSIM_NONE;
            for (uint32_t w = 0; w < nwaves; w++) {
                any |= sh.chk_any[par][w];
                ts = max(ts, sh.chk_max[par][w]);
                if (SKIP) { net = max(net, sh.chk_net[par][w]); nx = min(nx, sh.chk_nxt[par][w]); }
            }
            par ^= 1;
            if (!any) { done = true; break; }
            if (ts <= t - 1) { dead = true; t_dead = ts; break; }
            /* a task graph with an idle network: nothing is queued, staged
             * or about to be sent or activated, so no tick before the next
             * task finish can change any state; the tick loop goes there
             * directly (the identical state, only the clock advanced) */
            if (SKIP && net <= t - 1 && nx != MSIM_NONE && nx > t) {
                t = min(nx, t_end);
                slot = t % C.W;
                if (t >= t_end) break;
            }
        } else {
            __syncthreads();
        }
    }

    /* totals of this segment */
    uint64_t s0 = wave_sum_u64(a.hops), s1 = wave_sum_u64(a.delivered), s2 = wave_sum_u64(a.digest);
    uint32_t m0 = wave_max_u32(a.tmax), m1 = wave_max_u32(a.last_tx1), m2 = wave_max_u32(a.last_act1),
             m3 = wave_max_u32(a.max_arr), m4 = wave_max_u32(a.fault);
    if (lane == 0) {
        sh.sum[0][wave] = s0; sh.sum[1][wave] = s1; sh.sum[2][wave] = s2;
        sh.mx[0][wave] = m0; sh.mx[1][wave] = m1; sh.mx[2][wave] = m2; sh.mx[3][wave] = m3; sh.mx[4][wave] = m4;
    }
    __syncthreads();
    if (IN_LDS || split) {
        const uint4 *src = (const uint4 *)(lds + (IN_LDS ? rw_off : ro_hot));
        uint4 *dst = (uint4 *)(arena_g + rw_off);
        const uint32_t n = ((IN_LDS ? arena_bytes : rw_hot) - rw_off) / 16;
        for (uint32_t i = tid; i < n; i += nth) dst[i] = src[i];
    }
    if (tid == 0) finish_state(stp, sh, nwaves, t, done, dead, t_dead);
    __syncthreads();
}

/* ==================================================================== *
 * Compact path: one thread per port, port-private state in registers,
 * byte-row (SWAR) queue bookkeeping, shared state in LDS.
 * ==================================================================== */

/* A row of up to 16 byte counters held in registers (W words). */
template <int W>
struct Row {
    uint64_t w0, w1;
    __device__ __forceinline__ uint32_t get(uint32_t i) const
    {
        uint64_t w = (W == 1 || i < 8) ? w0 : w1;
        return (uint32_t)(w >> ((i & 7) * 8)) & 0xFFu;
    }
    __device__ __forceinline__ void set(uint32_t i, uint32_t v)
    {
        const uint32_t sh = (i & 7) * 8;
        const uint64_t m = ~(0xFFull << sh), b = (uint64_t)(v & 0xFFu) << sh;
        if (W == 1 || i < 8) w0 = (w0 & m) | b;
        else w1 = (w1 & m) | b;
    }
    __device__ __forceinline__ void load(const LDSP uint8_t *p)
    {
        w0 = *(const LDSP uint64_t *)p;
        w1 = W == 2 ? *(const LDSP uint64_t *)(p + 8) : 0ull;
    }
};

/* LDS-qualified pointers keep address arithmetic in 32 bits. */
template <typename DT>
struct CCtx {
    LDSP uint8_t *arr, *nslot, *pnxt;
    LDSP uint32_t *popped;     /* [2][nt], tick parity */
    const LDSP uint32_t *route;
    const LDSP DT *hout;
    const LDSP uint16_t *cgrp;
    const LDSP uint8_t *lidx;
    LDSP CRW2 *crw;
    LDSP uint64_t *fmask;      /* per switch ingress (slot - SB), slots its outputs returned */
    LDSP uint8_t *L;           /* the LDS image, and byte offsets of two of its arrays */
    uint32_t o_nslot, o_pnxt;
    const LDSP CGrp *grp;
    LDSP DT *pdesc, *sdesc;
    uint32_t *rec;
    uint32_t Q, W, R, n_flows, SB, nt, n_conn;
    uint32_t RP;               /* staging entries per (tick slot, port): R rounded up to 1, 2 or 4 */
    uint32_t S;                /* switch thread slots; pools are slot-major: [buffer slot][S] */
};

/* A collective group copied out of LDS in three 16-byte loads (the table
 * starts 16-byte aligned and a group is 48 bytes). */
__device__ __forceinline__ CGrp cgrp_load(const LDSP CGrp *p)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = ((const LDSP u32x4 *)p)[0], b = ((const LDSP u32x4 *)p)[1], c = ((const LDSP u32x4 *)p)[2];
    CGrp g;
    g.kind = (uint16_t)a.x; g.N = (uint16_t)(a.x >> 16); g.S = a.y; g.R = a.z; g.p = a.w;
    g.Xq = b.x; g.Xr = b.y; g.fid_base = b.z; g.conn_base = b.w; g.mS = c.x; g.link = c.y;
    return g;
}

/* Collective group of connection c. */
template <typename DT>
__device__ __forceinline__ CGrp cgrp_at(const CCtx<DT> &C, uint32_t c)
{
    return cgrp_load(C.grp + C.cgrp[c]);
}

/* Pool index of buffer slot s of the ingress in switch thread slot q (s < 64, S < 1024). */
template <typename DT>
__device__ __forceinline__ uint32_t cpool(const CCtx<DT> &C, uint32_t q, uint32_t s)
{
    return (s & 63u) * (C.S & 1023u) + q;   /* operands known to fit 24 bits: one full-rate multiply */
}

__device__ __forceinline__ uint32_t cdiv_S(const CGrp &g, uint32_t pos)
{
    return __umulhi(pos << 8, g.mS);
}

/* Chunk index rank i sends at step s (s < S): ring order, without division. */
__device__ __forceinline__ uint32_t cchunk(const CGrp &g, uint32_t i, uint32_t s)
{
    const uint32_t N = g.N;
    uint32_t v;
    if (g.kind == GK_RING_AG || s < N - 1) v = i + N - s;            /* in [1, 2N) */
    else v = i + 1 + N - (s - (N - 1));                              /* in [1, 2N] */
    if (v >= N) v -= N;
    if (v >= N) v -= N;
    return v;
}

/* F, the group kinds the code must handle, is fixed per kernel and per
 * experiment, so the kind tests below fold away where they cannot be true:
 *   0  rings only;
 *   1  rings, broadcasts and explicit flows;
 *   2  also trees, send/recv groups and gated rings. */
template <int F>
__device__ __forceinline__ uint32_t csize(const CGrp &g, uint32_t idx, uint32_t pos)
{
    if (F != 0 && g.kind == GK_BCAST) return g.p + (pos < g.Xq ? 1u : 0u);
    if (F == 2 && g.kind == GK_TREE) return pos + 1u < g.R ? g.p : g.Xq;
    if (F == 2 && g.kind == GK_SEQ) return g.p;
    const uint32_t r = cdiv_S(g, pos);
    if (r + 1 < g.R) return g.p;
    const uint32_t k = cchunk(g, idx, pos - __umul24(r, g.S));   /* r * S <= pos < 2^14 */
    return g.Xq + (k < g.Xr ? 1u : 0u);
}

template <int F>
__device__ __forceinline__ uint32_t cfid(const CGrp &g, uint32_t idx, uint32_t pos)
{
    if (F != 0 && g.kind == GK_XFLOW) return g.fid_base + idx;
    if (F != 0 && g.kind == GK_BCAST) return g.fid_base + idx * g.S + pos;
    if (F == 2 && g.kind == GK_TREE) return g.fid_base + pos * 2u * (g.N - 1u) + idx;
    if (F == 2 && g.kind == GK_SEQ) return g.fid_base + idx;
    return g.fid_base + __umul24(pos, g.N) + idx;               /* pos < 2^14, ring N <= 1024 */
}

template <int F>
__device__ __forceinline__ uint32_t cflows(const CGrp &g)
{
    if (F == 0) return g.R * g.S;
    if (F == 2 && g.kind == GK_TREE) return g.R;
    if (F == 2 && g.kind == GK_SEQ) return 1u;
    return g.kind == GK_BCAST ? g.S : (g.kind == GK_XFLOW ? 1u : g.R * g.S);
}

template <int F, typename DT>
__device__ __forceinline__ bool crecv_ok(const CCtx<DT> &C, const CGrp &g, uint32_t idx, uint32_t c, uint32_t pos)
{
    if (F == 0 || g.kind == GK_RING_AR || g.kind == GK_RING_AG) {
        if (pos - cdiv_S(g, pos) * g.S == 0) {
            /* a gated ring's first step waits for this rank's piece of its send/recv */
            if (F == 2 && pos == 0 && g.link != MSIM_NONE) return C.crw[C.grp[g.link].conn_base + idx].r_pos >= 1;
            return true;
        }
        const uint32_t cin = g.conn_base + (idx == 0 ? g.N - 1u : idx - 1u);
        return C.crw[cin].r_pos >= pos;
    }
    if (g.kind == GK_BCAST) return idx == 0 || C.crw[c - 1].r_pos > pos;
    /* send/recv: the previous receiver's copy has left the source */
    if (F == 2 && g.kind == GK_SEQ) return idx == 0 || (C.crw[c - 1].s_st & C_POS_MASK) >= 1;
    if (F == 2 && g.kind == GK_TREE)
        return tree_ready(g.N, idx, pos, [&](uint32_t j) { return (uint32_t)C.crw[g.conn_base + j].r_pos; });
    return true;
}

struct HostRegs {
    uint64_t ready;
    uint32_t pcnt, p0, p1, p2, p3;
};

template <int F, typename DT>
__device__ __forceinline__ void cactivate(const CCtx<DT> &C, Acc &a, HostRegs &hr, uint32_t c, uint32_t pos,
                                          const CGrp &g, uint32_t idx, uint32_t t)
{
    C.crw[c].s_st = (uint16_t)(pos | (CS_ACTIVE << C_STATE_SHIFT));
    if (F == 0 || g.kind != GK_XFLOW) C.crw[c].s_rem = (uint16_t)csize<F>(g, idx, pos);
    hr.ready |= 1ull << C.lidx[c];
    a.last_act1 = t + 1;
    if (C.rec) C.rec[C.n_flows + cfid<F>(g, idx, pos)] = t;
}

/* Activates connection d (of group g) if it was waiting and is now ready.
 * Every caller passes a connection whose source is the calling host. */
template <int F, typename DT>
__device__ __forceinline__ void cwake(const CCtx<DT> &C, Acc &a, HostRegs &hr, const CGrp &g, uint32_t d, uint32_t t)
{
    if ((C.crw[d].s_st >> C_STATE_SHIFT) != CS_IDLE) return;
    const uint32_t didx = d - g.conn_base, dpos = C.crw[d].s_st & C_POS_MASK;
    if (crecv_ok<F>(C, g, didx, d, dpos)) cactivate<F>(C, a, hr, d, dpos, g, didx, t);
}

/* After a flow over connection c (group g, index idx) has been fully
 * received: the connections leaving this host whose next flow waits on it. */
template <int F, typename DT>
__device__ __forceinline__ void cwake_dependents(const CCtx<DT> &C, Acc &a, HostRegs &hr, const CGrp &g, uint32_t idx,
                                                 uint32_t c, uint32_t t)
{
    if (F == 0 || g.kind == GK_RING_AR || g.kind == GK_RING_AG) {
        cwake<F>(C, a, hr, g, g.conn_base + (idx + 1u == g.N ? 0u : idx + 1u), t);
    } else if (g.kind == GK_BCAST) {
        if (idx + 1u < g.N) cwake<F>(C, a, hr, g, c + 1, t);
    } else if (F == 2 && g.kind == GK_SEQ) {
        /* this host's piece has arrived: its rank of every ring the send/recv gates */
        for (uint32_t k = 0; k < g.Xr; k++) {
            const CGrp h = cgrp_load(C.grp + g.link + k);
            cwake<F>(C, a, hr, h, h.conn_base + idx, t);
        }
    } else if (F == 2 && g.kind == GK_TREE) {
        tree_dependents(g.N, idx, [&](uint32_t j) { cwake<F>(C, a, hr, g, g.conn_base + j, t); });
    }
}

template <int F, typename DT>
__device__ __forceinline__ void ccheck(const CCtx<DT> &C, Acc &a, HostRegs &hr, uint32_t c, uint32_t t)
{
    const CGrp g = cgrp_at(C, c);
    const uint32_t idx = c - g.conn_base;
    const uint32_t pos = C.crw[c].s_st & C_POS_MASK;
    if (pos >= cflows<F>(g)) {
        C.crw[c].s_st = (uint16_t)(pos | (CS_DONE << C_STATE_SHIFT));
        /* a send/recv's next receiver waits on this send (its SEND predecessor) */
        if (F == 2 && g.kind == GK_SEQ && idx + 1u < g.N) cwake<F>(C, a, hr, g, c + 1, t);
    } else if (crecv_ok<F>(C, g, idx, c, pos)) {
        cactivate<F>(C, a, hr, c, pos, g, idx, t);
    } else {
        C.crw[c].s_st = (uint16_t)(pos | (CS_IDLE << C_STATE_SHIFT));
    }
}

/* A host's arrivals: deliveries, receive completions and the activations
 * they enable (phases A and B of the tick). */
template <int F, bool R1, typename DT>
__device__ __forceinline__ void chost_deliver(const CCtx<DT> &C, Acc &a, HostRegs &hr, LDSP DT *rec, uint32_t t)
{
    bool any = false;
    for (uint32_t k = 0; k < (R1 ? 1u : C.RP); k++) {
        const uint32_t e = rec[k];
        if (e == 0) break;
        any = true;
        const uint32_t c = (e - 1) >> DESC_SHIFT;
        LDSP CRW2 &cw = C.crw[c];
        a.delivered++;
        const uint32_t rem = cw.r_rem - 1u;
        cw.r_rem = (uint16_t)rem;
        if (rem) continue;
        const CGrp g = cgrp_at(C, c);
        const uint32_t idx = c - g.conn_base;
        uint32_t pos = cw.r_pos;
        const uint32_t fid = cfid<F>(g, idx, pos);
        a.digest += mix64(((uint64_t)fid << 32) | t);
        a.tmax = t;
        a.left--;
        if (C.rec) C.rec[fid] = t;
        pos++;
        cw.r_pos = (uint16_t)pos;
        if (pos < cflows<F>(g)) cw.r_rem = (uint16_t)csize<F>(g, idx, pos);
        cwake_dependents<F>(C, a, hr, g, idx, c, t);
    }
    /* at rate 1 the far output rewrites the entry every tick */
    if (!R1 && any)
        for (uint32_t k = 0; k < C.RP; k++) rec[k] = 0;
}

/* A host's pending activations (phase B): every connection at t = 0, then the
 * connections whose previous flow left during the last tick. */
template <int F, typename DT>
__device__ __forceinline__ void chost_pending(const CCtx<DT> &C, Acc &a, HostRegs &hr, const PortRO2 &pr, uint32_t t)
{
    if (t == 0) {
        for (uint32_t j = 0; j < pr.n_out; j++) ccheck<F>(C, a, hr, (uint32_t)C.hout[pr.vbase + j], t);
    } else if (hr.pcnt) {
        ccheck<F>(C, a, hr, hr.p0, t);
        if (hr.pcnt > 1) ccheck<F>(C, a, hr, hr.p1, t);
        if (hr.pcnt > 2) ccheck<F>(C, a, hr, hr.p2, t);
        if (hr.pcnt > 3) ccheck<F>(C, a, hr, hr.p3, t);
        hr.pcnt = 0;
    }
}

/* Connection cursors read in one 64-bit LDS access. */
__device__ __forceinline__ CRW2 crw_load(const LDSP CRW2 *p)
{
    const uint64_t v = *(const LDSP uint64_t *)p;
    CRW2 w;
    w.s_st = (uint16_t)v; w.s_rem = (uint16_t)(v >> 16); w.r_pos = (uint16_t)(v >> 32); w.r_rem = (uint16_t)(v >> 48);
    return w;
}

/* Makes the compiler hold v in a register at this point: a load above it is
 * complete here and is not sunk into a later branch, so loads pinned together
 * are waited for together. */
template <typename T>
__device__ __forceinline__ void pin(T &v)
{
    asm volatile("" : "+v"(v));
}

/* Rings only, rate 1: a host's arrivals and activations (phases A and B) for
 * t > 0, the same rules as chost_deliver<0> followed by chost_pending<0>.
 * At rate 1 at most one packet arrives per tick, and at most one flow left
 * the NIC during the last tick.  So at most two connections leaving this host
 * may start a flow now: the ring successor d of a connection c whose flow was
 * fully received now (d's receive predecessor is that flow), and the pending
 * connection p whose flow finished sending (its send predecessor).  The reads
 * are issued in three rounds instead of one dependent access at a time.
 * Rank i's connection of a ring receives from connection (i - 1) mod N of the
 * same group, so d is c + 1 unless c is the group's last rank. */
template <typename DT>
__device__ __forceinline__ void chost_ring_r1(const CCtx<DT> &C, Acc &a, HostRegs &hr, LDSP DT *rec, uint32_t t)
{
    const bool pend = hr.pcnt != 0;
    if (hr.pcnt > 1) a.fault = 1;
    hr.pcnt = 0;
    const uint32_t p = pend ? hr.p0 : 0u;
    /* round 1: the arrival, and the pending connection's send state and group
     * (the delivery below writes receive-side fields only) */
    uint32_t e = rec[0];
    uint32_t p_st = C.crw[p].s_st, p_gi = C.cgrp[p], p_li = C.lidx[p];
    pin(e); pin(p_st); pin(p_gi); pin(p_li);
    const bool got = e != 0;
    const uint32_t c = got ? (e - 1) >> DESC_SHIFT : 0u;
    const uint32_t c1 = c + 1u < C.n_conn ? c + 1u : c;
    /* round 2: c's cursors and group, the send state of c + 1, p's group */
    uint64_t cw = *(const LDSP uint64_t *)(C.crw + c);
    uint32_t gi = C.cgrp[c];
    uint32_t n_st = C.crw[c1].s_st, n_li = C.lidx[c1];
    CGrp h = cgrp_load(C.grp + p_gi);
    pin(cw); pin(gi); pin(n_st); pin(n_li);
    pin(h.kind); pin(h.N); pin(h.S); pin(h.R); pin(h.p); pin(h.Xq); pin(h.Xr); pin(h.fid_base); pin(h.conn_base); pin(h.mS);
    const uint32_t hN = h.N, hS = h.S, hR = h.R, hcb = h.conn_base;
    const uint32_t r_pos = (uint32_t)(cw >> 32) & 0xFFFFu, r_rem = (uint32_t)(cw >> 48);
    const bool fin = got && r_rem == 1u;            /* c's flow is now fully received */
    const uint32_t pidx = p - hcb, ppos = p_st & C_POS_MASK;
    const uint32_t cin = hcb + (pidx == 0 ? hN - 1u : pidx - 1u);
    /* round 3: c's group in full, the receive position of p's predecessor */
    CGrp g;
    uint32_t cin_rpos = 0;
    if (pend) cin_rpos = C.crw[cin].r_pos;
    if (fin) g = cgrp_load(C.grp + gi);
    pin(cin_rpos);
    if (got) a.delivered++;
    if (got && !fin) C.crw[c].r_rem = (uint16_t)(r_rem - 1u);
    uint32_t d = MSIM_NONE, rpos = 0;
    if (fin) {
        const uint32_t idx = c - g.conn_base;
        const uint32_t fid = cfid<0>(g, idx, r_pos);
        a.tmax = t;
        a.left--;
        if (C.rec) C.rec[fid] = t;
        rpos = r_pos + 1u;
        const uint32_t nrem = rpos < __umul24(g.R, g.S) ? csize<0>(g, idx, rpos) : 0u;
        *(LDSP uint32_t *)&C.crw[c].r_pos = rpos | (nrem << 16);
        d = idx + 1u == g.N ? c + 1u - g.N : c + 1u;
        if (d != c1) {                              /* c is the last rank: one more round */
            n_st = C.crw[d].s_st;
            n_li = C.lidx[d];
        }
        a.digest += mix64(((uint64_t)fid << 32) | t);
    }
    /* d waits for its receive predecessor, the flow over c, received through rpos */
    if (fin && (n_st >> C_STATE_SHIFT) == CS_IDLE) {
        const uint32_t dpos = n_st & C_POS_MASK;
        if (dpos - __umul24(cdiv_S(g, dpos), g.S) == 0 || rpos >= dpos) {
            const uint32_t didx = d - g.conn_base;
            *(LDSP uint32_t *)&C.crw[d].s_st = (dpos | (CS_ACTIVE << C_STATE_SHIFT)) | (csize<0>(g, didx, dpos) << 16);
            hr.ready |= 1ull << n_li;
            a.last_act1 = t + 1;
            if (C.rec) C.rec[C.n_flows + cfid<0>(g, didx, dpos)] = t;
        }
    }
    if (pend) {
        if (ppos >= __umul24(hR, hS)) {
            C.crw[p].s_st = (uint16_t)(ppos | (CS_DONE << C_STATE_SHIFT));
        } else {
            /* cin's receive position as of now: c's, if this tick completed it */
            const uint32_t rp = (fin && cin == c) ? rpos : cin_rpos;
            if (ppos - __umul24(cdiv_S(h, ppos), hS) == 0 || rp >= ppos) {
                *(LDSP uint32_t *)&C.crw[p].s_st = (ppos | (CS_ACTIVE << C_STATE_SHIFT)) | (csize<0>(h, pidx, ppos) << 16);
                hr.ready |= 1ull << p_li;
                a.last_act1 = t + 1;
                if (C.rec) C.rec[C.n_flows + cfid<0>(h, pidx, ppos)] = t;
            } else {
                C.crw[p].s_st = (uint16_t)(ppos | (CS_IDLE << C_STATE_SHIFT));
            }
        }
    }
}

/* Stages the m-th packet this output sends in tick t for arrival at t + delay:
 * entry m of the far port's record for that tick slot holds desc + 1 (0 means
 * empty), so the sender never reads the record. */
/* Packet-hops are counted from the output's pushed total, and the latest
 * arrival tick from its last transmission plus its fixed delay. */
template <typename DT>
__device__ __forceinline__ void ctransmit(const CCtx<DT> &C, Acc &a, uint32_t desc, uint32_t t, uint32_t dst)
{
    C.sdesc[dst] = (DT)(desc + 1);
    a.last_tx1 = t + 1;
}

/* Keeps the compiler from moving LDS accesses across a phase boundary.  Lanes
 * of one switch talk through LDS inside a tick; the LDS executes a wavefront's
 * instructions in issue order, so no hardware wait is needed, only program
 * order. */
__device__ __forceinline__ void wave_lds_fence()
{
    asm volatile("" ::: "memory");
}

/*
 * One tick t of a compact experiment, per wavefront, with one workgroup
 * barrier at its end:
 *   arrivals    switch ingress: zeroes its pop count for tick t, then the
 *               packets with arrival tick t join their queue, in slots taken
 *               from its free mask; host: deliveries, then activations
 *               (Schedule);
 *   forwarding  every output pulls, up to its rate, while credit lasts (the
 *               far ingress's pops through t-1, added up tick by tick); each
 *               pop returns its slot to the ingress's free word and counts in
 *               the ingress's pop count for tick t.
 * Arrivals read staging written at least one barrier earlier (delay >= 1);
 * forwarding reads queues filled by the arrivals of the same switch (same
 * wavefront), and the slots it returns are taken again from the next tick on.
 */
template <int W, typename DT, bool R1, bool X>
__device__ void run_compact(const KParams &kp, uint32_t x, uint8_t *arena_g, uint8_t *lds, Shared &sh)
{
    const uint32_t tid = threadIdx.x, nth = blockDim.x;
    const uint32_t lane = tid & 63, wave = tid >> 6, nwaves = (nth + 63) >> 6;
    ExpState *stp = (ExpState *)(kp.ws + kp.o_state) + x;
    const ArenaHdr2 *H = (const ArenaHdr2 *)arena_g;
    const uint32_t lds_bytes = H->lds_bytes, rw_off = H->rw_off;
    {
        const uint4 *src = (const uint4 *)arena_g;
        uint4 *dst = (uint4 *)lds;
        for (uint32_t i = tid; i < lds_bytes / 16; i += nth) dst[i] = src[i];
    }
    const uint32_t nt = H->nt, nh = H->H, SB = H->SB;
    const bool used = tid < nt;
    PortRO2 pr = {};
    PortPriv pv = {};
    if (used) {
        pr = ((const PortRO2 *)(arena_g + H->o_port))[tid];
        pv = ((const PortPriv *)(arena_g + H->o_priv))[tid];
    }
    LDSP uint8_t *L = (LDSP uint8_t *)lds;
    CCtx<DT> C;
    C.arr = L + H->o_arr;
    C.nslot = L + H->o_nslot;
    C.pnxt = L + H->o_pnxt;
    C.popped = (LDSP uint32_t *)(L + H->o_popped);
    C.route = (const LDSP uint32_t *)(L + H->o_route);
    C.hout = (const LDSP DT *)(L + H->o_hout);
    C.cgrp = (const LDSP uint16_t *)(L + H->o_cgrp);
    C.lidx = (const LDSP uint8_t *)(L + H->o_lidx);
    C.crw = (LDSP CRW2 *)(L + H->o_crw);
    C.fmask = (LDSP uint64_t *)(L + H->o_fmask);
    C.L = L;
    C.o_nslot = H->o_nslot;
    C.o_pnxt = H->o_pnxt;
    C.grp = (const LDSP CGrp *)(L + H->o_grp);
    C.pdesc = (LDSP DT *)(L + H->o_pdesc);
    C.sdesc = (LDSP DT *)(L + H->o_sdesc);
    C.Q = H->Q;
    C.W = H->W;
    C.R = H->R;
    C.n_flows = H->n_flows;
    C.n_conn = H->n_conn;
    C.SB = SB;
    C.nt = nt;
    C.RP = R1 ? 1u : (H->R <= 1 ? 1u : (H->R <= 2 ? 2u : 4u));
    C.S = nt - SB;
    uint64_t roff = ((const uint64_t *)(kp.ws + kp.o_rec_off))[x];
    C.rec = roff == ~0ull ? nullptr : (uint32_t *)(kp.ws + roff);

    const bool rings_only = (H->flags & AF_RINGS_ONLY) != 0;   /* uniform: one experiment per workgroup */
    const bool is_host = tid < nh && (pr.flags & PF_USED);
    const bool is_sw = tid >= SB && (pr.flags & PF_USED);
    const bool alive = pr.flags & PF_ALIVE;
    const bool peer_host = pr.flags & PF_PEER_HOST;
    constexpr uint32_t RSZ = 8u * W;              /* bytes per VOQ row: one per input port */
    const uint32_t deg = pr.deg, local = pr.local, Q = C.Q;
    uint64_t freem = pv.freem;                     /* switch ingress: free buffer slots */
    uint32_t popped = pv.popped, pushed = pv.pushed, rr = pv.rr;
    HostRegs hr;
    hr.ready = pv.ready;
    hr.pcnt = pv.pcnt;
    hr.p0 = pv.pend[0]; hr.p1 = pv.pend[1]; hr.p2 = pv.pend[2]; hr.p3 = pv.pend[3];
    const uint32_t pool = is_sw ? tid - SB : 0;   /* buffer slot s of this ingress: pool + s * C.S */
    const bool q32 = Q <= 32;                      /* free-slot mask fits one 32-bit word */
    const uint32_t qbase = tid - local;          /* thread slot of this switch's port 0 */
    const uint32_t rowp = pr.vbase + local * RSZ;
    /* staging: the record of (tick slot, port) starts at slot * tstride + port * RP */
    const uint32_t RP = C.RP, tstride = nt * RP, wsz = C.W * tstride;
    const uint32_t doff = pr.delay * tstride, poff = pr.peer * RP, myoff = tid * RP;
    const uint32_t pushed0 = pushed;               /* packet-hops of this run: pushed - pushed0 */

    Acc a;
    a.hops = a.delivered = a.digest = 0;
    a.tmax = a.last_tx1 = a.last_act1 = a.max_arr = 0;
    a.left = is_host ? pv.left : 0;
    a.fault = 0;
    if (tid == 0) { sh.chk_any[0][0] = sh.chk_any[1][0] = 0; sh.chk_max[0][0] = sh.chk_max[1][0] = 0; }
    __syncthreads();

    const uint32_t t0 = stp->t_now;
    const uint32_t t_end = (uint64_t)t0 + kp.max_ticks > 0xFFFFFFF0ull ? 0xFFFFFFF0u : t0 + kp.max_ticks;
    const uint32_t hist = max(max(stp->last_tx1, stp->last_act1), stp->max_arr);
    uint32_t t = t0, par = 0, sb = (t0 % C.W) * tstride, tp = (t0 & 1u) ? nt : 0u;
    bool done = false, dead = false;
    uint32_t t_dead = 0;
    while (t < t_end) {
        /* ---------------- arrivals */
        if (is_sw) {
            /* this tick's pop count starts at zero; the outputs of this switch
             * add to it while they forward, and the far outputs read it during
             * tick t+1.  At most RP packets arrive per ingress and tick. */
            C.popped[tp + tid] = 0;
            LDSP DT *rec = C.sdesc + sb + myoff;
            /* one arriving packet: e = descriptor + 1, the same packet with its
             * hop index advanced */
            auto arrive = [&](uint32_t e) {
                const uint32_t desc = e - 1;
                const uint32_t c = desc >> DESC_SHIFT, hop = desc & DESC_HOP_MASK;
                const uint32_t o = (C.route[c] >> (4 * hop)) & 0xFu;
                const uint32_t vq = pr.vbase + o * RSZ + local;   /* queue (this input, o) */
                const uint32_t head = C.nslot[vq], tail = C.arr[vq];
                /* free slots: the register mask, refilled from the slots the
                 * outputs returned only when it runs dry */
                if (freem == 0)
                    freem = __hip_atomic_exchange(C.fmask + pool, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (freem == 0 || o >= deg) {
                    a.fault = 1;
                    return;
                }
                uint32_t s;
                if (q32) {
                    const uint32_t lo = (uint32_t)freem;
                    s = __builtin_ctz(lo);
                    freem = lo & (lo - 1u);
                } else {
                    s = __builtin_ctzll(freem);
                    freem &= freem - 1;
                }
                C.pdesc[cpool(C, pool, s)] = (DT)e;
                /* an empty queue has the head byte Q_EMPTY: the new slot
                 * becomes its head, else it goes behind the tail */
                const uint32_t at_head = C.o_nslot + vq, at_tail = C.o_pnxt + cpool(C, pool, tail);
                C.L[head == Q_EMPTY ? at_head : at_tail] = (uint8_t)s;
                C.arr[vq] = (uint8_t)s;
            };
            if (R1) {
                /* the feeding output rewrites its entry every tick */
                const uint32_t e = rec[0];
                if (e != 0) arrive(e);
            } else {
                /* the RP (2 or 4) entries of the record in one read; they fill
                 * in order, and the reader clears what was staged */
                uint32_t e4[4];
                if (C.RP == 1) {
                    e4[0] = rec[0]; e4[1] = e4[2] = e4[3] = 0;
                } else if (sizeof(DT) == 2 && C.RP == 2) {
                    const uint32_t w = *(const LDSP uint32_t *)rec;
                    e4[0] = w & 0xFFFFu; e4[1] = w >> 16; e4[2] = e4[3] = 0;
                } else if (sizeof(DT) == 2) {
                    const uint64_t w = *(const LDSP uint64_t *)rec;
                    e4[0] = (uint32_t)w & 0xFFFFu; e4[1] = (uint32_t)w >> 16;
                    e4[2] = (uint32_t)(w >> 32) & 0xFFFFu; e4[3] = (uint32_t)(w >> 48);
                } else if (C.RP == 2) {
                    const uint64_t w = *(const LDSP uint64_t *)rec;
                    e4[0] = (uint32_t)w; e4[1] = (uint32_t)(w >> 32); e4[2] = e4[3] = 0;
                } else {
                    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                    const u32x4 w = *(const LDSP u32x4 *)rec;
                    e4[0] = w.x; e4[1] = w.y; e4[2] = w.z; e4[3] = w.w;
                }
#pragma unroll
                for (uint32_t k = 0; k < 4; k++)
                    if (e4[k] != 0) arrive(e4[k]);
                if (e4[0] != 0) {
                    if (C.RP * sizeof(DT) == 4) *(LDSP uint32_t *)rec = 0u;
                    else if (C.RP * sizeof(DT) == 8) *(LDSP uint64_t *)rec = 0ull;
                    else for (uint32_t k = 0; k < C.RP; k++) rec[k] = 0;
                }
            }
        } else if (is_host) {
            LDSP DT *rec = C.sdesc + sb + myoff;
            /* the ring-only copy costs registers the faster-link kinds do not have */
            if (R1 && !X && rings_only) {
                if (t != 0) {
                    chost_ring_r1(C, a, hr, rec, t);
                } else {
                    chost_deliver<0, R1>(C, a, hr, rec, t);
                    chost_pending<0>(C, a, hr, pr, t);
                }
            } else {
                chost_deliver<X ? 2 : 1, R1>(C, a, hr, rec, t);
                chost_pending<X ? 2 : 1>(C, a, hr, pr, t);
            }
        }
        wave_lds_fence();
        /* ---------------- forwarding */
        uint32_t dst = sb + doff;
        if (dst >= wsz) dst -= wsz;
        dst += poff;
        if (is_sw && alive) {
            /* up to rate grants, each cyclic from rr over the non-empty queues
             * toward this output, read from its row of head bytes; the credit
             * counts the far ingress's pops through t-1 */
            if (!peer_host) popped += C.popped[(tp ^ nt) + pr.peer];
            int32_t credit = peer_host ? (int32_t)pr.rate : (int32_t)Q - (int32_t)(pushed - popped);
            Row<W> hrow, trow;
            hrow.load(C.nslot + rowp);
            trow.load(C.arr + rowp);
            const uint64_t F = 0x8080808080808080ull;          /* a slot byte < 64 has bit 7 clear */
            uint32_t out = 0;                                          /* rate 1: staged entry, desc + 1 or 0 */
            /* a loop count the whole wavefront shares (the largest rate), each
             * lane's rate and credit as guards: no per-lane loop exits */
            for (uint32_t m = 0; m < (R1 ? 1u : C.RP); m++) {
                if (!R1 && (m >= pr.rate || credit <= 0)) continue;
                if (R1 && credit <= 0) continue;
                const int i = first_from<W>(~hrow.w0 & F, W == 2 ? (~hrow.w1 & F) : 0ull, rr);
                if (i < 0) continue;
                const uint32_t vq = rowp + (uint32_t)i;                 /* queue (i, this output) */
                const uint32_t qpool = qbase + (uint32_t)i - SB;
                const uint32_t s = hrow.get((uint32_t)i);
                const uint32_t desc = C.pdesc[cpool(C, qpool, s)];
                const uint32_t next = C.pnxt[cpool(C, qpool, s)];
                /* popping the tail empties the queue */
                const uint32_t nh = s == trow.get((uint32_t)i) ? Q_EMPTY : next;
                C.nslot[vq] = (uint8_t)nh;
                if (!R1) hrow.set((uint32_t)i, nh);
                /* the slot goes back to the ingress and the pop into its count
                 * for this tick (other outputs of this switch may hit the same
                 * ingress in the same instruction) */
                __hip_atomic_fetch_or(C.fmask + qpool, 1ull << s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(C.popped + tp + qbase + (uint32_t)i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                rr = (uint32_t)i + 1 == deg ? 0 : (uint32_t)i + 1;
                if (R1) {
                    out = desc + 1;
                    a.last_tx1 = t + 1;
                } else {
                    ctransmit(C, a, desc, t, dst + m);
                }
                pushed++;
                credit--;
            }
            /* written every tick, so the far ingress never clears what it read */
            if (R1) C.sdesc[dst] = (DT)out;
        } else if (is_host && alive && pr.n_out) {
            popped += C.popped[(tp ^ nt) + pr.peer];
            int32_t credit = (int32_t)Q - (int32_t)(pushed - popped);
            uint32_t out = 0;      /* rate 1: the staged entry, written every tick (0 when idle) */
            for (uint32_t m = 0; m < (R1 ? 1u : pr.rate) && credit > 0 && hr.ready; m++) {
                const uint64_t rot = rr ? (hr.ready >> rr) | (hr.ready << (64 - rr)) : hr.ready;
                const uint32_t j = (rr + (uint32_t)__builtin_ctzll(rot)) & 63u;
                const uint32_t c = C.hout[pr.vbase + j];
                if (R1) {
                    out = (c << DESC_SHIFT) + 1u;
                    a.last_tx1 = t + 1;
                } else {
                    ctransmit(C, a, c << DESC_SHIFT, t, dst + m);
                }
                pushed++;
                credit--;
                rr = j + 1 == pr.n_out ? 0 : j + 1;
                LDSP CRW2 &cw = C.crw[c];
                const uint32_t rem = cw.s_rem - 1u;
                cw.s_rem = (uint16_t)rem;
                if (rem == 0) {
                    hr.ready &= ~(1ull << j);
                    const uint32_t pos = cw.s_st & C_POS_MASK;
                    if (C.rec) {
                        const CGrp g = cgrp_at(C, c);
                        C.rec[2 * C.n_flows + cfid<X ? 2 : 1>(g, c - g.conn_base, pos)] = t + 1;
                    }
                    cw.s_st = (uint16_t)(pos + 1);
                    /* append c to the pending list (selects, not branches); at
                     * rate 1 the list holds one entry at most */
                    if (R1) {
                        hr.p0 = c;
                        hr.pcnt = 1;
                    } else {
                        hr.p0 = hr.pcnt == 0 ? c : hr.p0;
                        hr.p1 = hr.pcnt == 1 ? c : hr.p1;
                        hr.p2 = hr.pcnt == 2 ? c : hr.p2;
                        hr.p3 = hr.pcnt == 3 ? c : hr.p3;
                        hr.pcnt++;
                    }
                }
            }
            if (R1) C.sdesc[dst] = (DT)out;
        }
        wave_lds_fence();
        t++;
        sb += tstride;
        if (sb == wsz) sb = 0;
        tp ^= nt;
        if (((t - t0) & ((t - t0) < CHECK_LONG ? CHECK_EVERY - 1u : CHECK_EVERY_LONG - 1u)) == 0 || t == t_end) {
            a.max_arr = a.last_tx1 ? a.last_tx1 - 1 + pr.delay : 0;
            uint32_t any = __ballot(a.left > 0) != 0ull;
            uint32_t ts = wave_max_u32(max(max(a.last_tx1, a.last_act1), a.max_arr));
            /* one word per reduction, updated by one lane per wavefront; the
             * other parity's words are cleared for the next check, which
             * comes at least one barrier later */
            if (lane == 0) {
                if (any) atomicOr(&sh.chk_any[par][0], 1u);
                atomicMax(&sh.chk_max[par][0], ts);
            }
            __syncthreads();
            any = sh.chk_any[par][0];
            ts = max(hist, sh.chk_max[par][0]);
            if (tid == 0) { sh.chk_any[par ^ 1][0] = 0; sh.chk_max[par ^ 1][0] = 0; }
            par ^= 1;
            if (!any) { done = true; break; }
            if (ts <= t - 1) { dead = true; t_dead = ts; break; }
        } else {
            __syncthreads();
        }
    }

    /* one launch runs at most 2^30 ticks, so a port at rate <= 4 pushes fewer than 2^32 packets */
    a.hops = pushed - pushed0;
    a.max_arr = a.last_tx1 ? a.last_tx1 - 1 + pr.delay : 0;

    /* write back: shared mutable image, registers, totals */
    {
        const uint4 *src = (const uint4 *)(lds + rw_off);
        uint4 *dst = (uint4 *)(arena_g + rw_off);
        for (uint32_t i = tid; i < (lds_bytes - rw_off) / 16; i += nth) dst[i] = src[i];
    }
    if (used) {
        pv = PortPriv{};
        pv.freem = freem;
        pv.popped = popped; pv.pushed = pushed; pv.rr = rr;
        pv.ready = hr.ready; pv.pcnt = hr.pcnt;
        pv.pend[0] = hr.p0; pv.pend[1] = hr.p1; pv.pend[2] = hr.p2; pv.pend[3] = hr.p3;
        pv.left = is_host ? a.left : 0;
        ((PortPriv *)(arena_g + H->o_priv))[tid] = pv;
    }
    uint64_t s0 = wave_sum_u64(a.hops), s1 = wave_sum_u64(a.delivered), s2 = wave_sum_u64(a.digest);
    uint32_t m0 = wave_max_u32(a.tmax), m1 = wave_max_u32(a.last_tx1), m2 = wave_max_u32(a.last_act1),
             m3 = wave_max_u32(a.max_arr), m4 = wave_max_u32(a.fault);
    if (lane == 0) {
        sh.sum[0][wave] = s0; sh.sum[1][wave] = s1; sh.sum[2][wave] = s2;
        sh.mx[0][wave] = m0; sh.mx[1][wave] = m1; sh.mx[2][wave] = m2; sh.mx[3][wave] = m3; sh.mx[4][wave] = m4;
    }
    __syncthreads();
    if (tid == 0) finish_state(stp, sh, nwaves, t, done, dead, t_dead);
    __syncthreads();
}

/* ==================================================================== *
 * Ring path: rings only (at most 10 ranks), every link at rate 1, switches
 * of at most 8 ports, buffers of at most 16 packets (the ring format of
 * msim_layout.h).
 *
 * One thread per port and one workgroup barrier per tick, as on the compact
 * path.  With a dozen wavefronts sharing a CU's four SIMDs, the tick is bound
 * by the vector instructions all of them issue (every wavefront runs each
 * branch any of its lanes needs), so this path is built to keep that count
 * low:
 *   - a host's flow events touch one 16-byte pair record it alone owns and
 *     the ring-channel record the arriving descriptor names, read in two
 *     rounds; the last-round chunk sizes come from a precomputed bit mask;
 *   - a switch ingress keeps its queues' tails, non-empty bits and free slots
 *     in registers, and takes the egress from the descriptor, which carries
 *     the remaining route;
 *   - a switch output finds its candidates in an 8-bit word of non-empty
 *     inputs, pops from the head slot row, and hands the freed slot (and an
 *     emptied queue) back to the ingress with one LDS atomic OR into a word
 *     of this tick's parity.  At the next tick's first read round the
 *     ingress folds that word into its registers and the port feeding it
 *     counts its slot bits as pops for its credit; the ingress clears the
 *     word a tick later, before its outputs write it again;
 *   - hosts queue each received (flow, RD) word in LDS, and a wavefront
 *     mixes every host's queue into the digest together once one is full;
 *   - host, switch and empty wavefronts run separate copies of the tick loop
 *     (same barriers), and when every delay is 1 ticks run in even/odd pairs
 *     so every staging and hand-back address is a loop constant.
 * The atomic ORs are the one many-to-one write: up to 8 outputs of a switch
 * may hand back slots of the same ingress, or mark the same output's word,
 * in one instruction.  OR is order-independent, so results do not depend on
 * the order the LDS applies them.
 * ==================================================================== */

/* First set bit of mask (nonzero) at or after bit rr, cyclically over 32 bits. */
__device__ __forceinline__ uint32_t first_ready(uint32_t mask, uint32_t rr)
{
    const uint32_t rot = __builtin_amdgcn_alignbit(mask, mask, rr);   /* mask rotated right by rr */
    return (rr + (uint32_t)__builtin_ctz(rot | (rot == 0 ? 1u : 0u))) & 31u;
}

/* Packets of the flow at position pos of the connection whose rank r gives
 * r2N = r + 2N: p in every round but the last; in the last round the chunk
 * (r - step) mod N holds Xq plus bit r + 2N - step of T. */
__device__ __forceinline__ uint32_t rsize(const RGrp &g, uint32_t r2N, uint32_t pos)
{
    const uint32_t T1 = g.RS - g.S;
    return pos < T1 ? g.p : g.Xq + ((g.T >> (r2N - (pos - T1))) & 1u);
}

__device__ __forceinline__ uint32_t rfid(const RGrp &g, uint32_t r, uint32_t pos)
{
    return g.fid_base + __umul24(pos, g.N) + r;  /* pos < 2^14, N <= 10 */
}

__device__ __forceinline__ RGrp rgrp_load(const LDSP RGrp *p)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = ((const LDSP u32x4 *)p)[0], b = ((const LDSP u32x4 *)p)[1];
    RGrp g;
    g.fid_base = a.x; g.N = a.y; g.S = a.z; g.RS = a.w; g.p = b.x; g.Xq = b.y; g.T = b.z; g.mS = b.w;
    return g;
}

__device__ __forceinline__ RPair rpair_load(const LDSP RPair *p)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 a = *(const LDSP u32x4 *)p;
    RPair r;
    r.snd = a.x; r.rcv = a.y; r.desc = a.z; r.gi = a.w;
    return r;
}

#define RP_REM(w) ((w) & 0xFFFFu)
#define RP_POS(w) (((w) >> 16) & C_POS_MASK)
#define RP_ST(w) ((w) >> 30)
#define GI_GRP(w) ((w) & 1023u)
#define GI_RANK(w) (((w) >> 10) & 1023u)
#define GI_PRED(w) ((w) >> 20)

__device__ void run_ring(const KParams &kp, uint32_t x, uint8_t *arena_g, uint8_t *lds, Shared &sh)
{
    const uint32_t tid = threadIdx.x, nth = blockDim.x;
    const uint32_t lane = tid & 63, wave = tid >> 6, nwaves = (nth + 63) >> 6;
    ExpState *stp = (ExpState *)(kp.ws + kp.o_state) + x;
    const ArenaHdr3 *H = (const ArenaHdr3 *)arena_g;
    const uint32_t lds_bytes = H->lds_bytes, rw_off = H->rw_off;
    {
        const uint4 *src = (const uint4 *)arena_g;
        uint4 *dst = (uint4 *)lds;
        for (uint32_t i = tid; i < lds_bytes / 16; i += nth) dst[i] = src[i];
    }
    const uint32_t nt = H->nt, SB = H->SB, Q = H->Q, W = H->W, n_flows = H->n_flows;
    const uint32_t S = nt - SB;                      /* switch slots: pool stride */
    const uint32_t FWS = S + 1;                      /* one half of fw; word S of each half stays 0 */
    LDSP uint8_t *L = (LDSP uint8_t *)lds;
    const LDSP RGrp *grp = (const LDSP RGrp *)(L + H->o_grp);
    LDSP RPair *pair = (LDSP RPair *)(L + H->o_pair);
    LDSP uint32_t *pdesc = (LDSP uint32_t *)(L + H->o_pdesc);
    LDSP uint8_t *pnxt = L + H->o_pnxt;
    LDSP uint8_t *head = L + H->o_head;
    LDSP uint32_t *nzw = (LDSP uint32_t *)(L + H->o_nzw);
    LDSP uint32_t *fw = (LDSP uint32_t *)(L + H->o_fw);
    LDSP uint32_t *sdesc = (LDSP uint32_t *)(L + H->o_sdesc);
    /* a host's received flows not yet mixed into its digest (host lanes only) */
    LDSP uint64_t *dq = (LDSP uint64_t *)(L + H->o_dq) + (tid < SB ? tid : 0u) * RING_DQ;
    uint64_t roff = ((const uint64_t *)(kp.ws + kp.o_rec_off))[x];
    uint32_t *rec = roff == ~0ull ? nullptr : (uint32_t *)(kp.ws + roff);

    const bool used = tid < nt;
    RingPort pr = {};
    RingPriv pv = {};
    if (used) {
        pr = ((const RingPort *)(arena_g + H->o_port))[tid];
        pv = ((const RingPriv *)(arena_g + H->o_priv))[tid];
    }
    const bool is_host = (pr.flags & (PF_USED | PF_HOST)) == (PF_USED | PF_HOST);
    const bool is_sw = (pr.flags & (PF_USED | PF_HOST)) == PF_USED;
    const bool alive = pr.flags & PF_ALIVE;
    const bool peer_host = pr.flags & PF_PEER_HOST;
    const bool buffered = alive && !peer_host;                 /* its output feeds a switch buffer */
    /* the credit bound of this port's output: Q toward a switch buffer, none
     * toward a host, nothing over a failed cable */
    const uint32_t qcap = !alive ? 0u : buffered ? Q : 0xFFFFFFFFu;
    /* the fw word of the buffer this port's output feeds (word S: always 0) */
    const uint32_t peer_pool = buffered ? pr.peer - SB : S;
    const uint32_t local = pr.local;
    const uint32_t n_out = is_host ? pr.row : 0u;
    const uint32_t row = is_sw ? pr.row + local : 0u;          /* this port's switch row */
    const uint32_t pool = is_sw ? tid - SB : S;                /* this ingress's buffer pool */
    const uint32_t pool0 = is_sw ? tid - local - SB : 0u;      /* pool of its switch's port 0 */
    const uint32_t hb0 = pr.row * 8u + local;                  /* head byte of queue (this ingress -> output 0) */
    /* staging: tick slots of NS words; this lane's word is pr.stg, its far
     * end's pr.pstg (a permutation of the slots under which every wavefront
     * reads, and writes, 64 different LDS banks) */
    const uint32_t NS = (nt + 63) & ~63u;
    const uint32_t doff = pr.delay * NS, wsz = W * NS;
    /* this ingress's buffer slot s: pd_me + s * S words, pn_me + s * S bytes */
    LDSP uint8_t *const pd_me = (LDSP uint8_t *)(pdesc + pool);
    LDSP uint8_t *const pn_me = pnxt + pool;
    const uint32_t S4 = S * 4u;
    uint32_t pushed = pv.pushed, rr = pv.rr, mask = pv.mask, tails = pv.tails, ne = pv.ne, seen = pv.seen;
    const uint32_t pushed0 = pushed;

    uint32_t delivered = 0, tmax = 0, last_tx1 = 0, last_act1 = 0, fault = 0;
    uint64_t digest = 0;
    uint32_t fmin = ~0u;                                       /* least free-slot mask an arrival met */
    uint32_t qn = 0;                                           /* entries in this host's digest queue */
    uint32_t last_w = 0;                                       /* switch wavefront, every delay 1: last send + 1 */
    /* mix the queued (flow, RD) words of every host of the wavefront at once:
     * one pass over RING_DQ entries instead of one mix per tick with an
     * arrival somewhere in the wavefront */
    auto flush_digest = [&]() {
#pragma unroll
        for (uint32_t k = 0; k < RING_DQ; k++) {
            const uint64_t z = dq[k];
            if (k < qn) digest += mix64(z);
        }
        qn = 0;
    };
    uint32_t left = is_host ? tails : 0u;
    __syncthreads();

    const uint32_t t0 = stp->t_now;
    const uint32_t t_end = (uint64_t)t0 + kp.max_ticks > 0xFFFFFFF0ull ? 0xFFFFFFF0u : t0 + kp.max_ticks;
    const uint32_t hist = max(max(stp->last_tx1, stp->last_act1), stp->max_arr);
    /* every pair's first flow is active from tick 0 (the initial image says so) */
    if (t0 == 0 && is_host && n_out) {
        last_act1 = 1;
        if (rec)
            for (uint32_t k = 0; k < n_out; k++) {
                const uint32_t gi = pair[k * SB + tid].gi;
                rec[n_flows + rfid(rgrp_load(grp + GI_GRP(gi)), GI_RANK(gi), 0)] = 0;
            }
    }
    LDSP RPair *pair_me = pair + tid;                          /* a host's pair records */
    uint32_t t = t0, par = 0, sb = (t0 % W) * NS;
    bool done = false, dead = false;
    uint32_t t_dead = 0;
    /* the next tick at whose end the workgroup checks for completion */
    auto next_check = [&]() -> uint32_t {
        const uint32_t d = t - t0;
        const uint32_t nd = d < CHECK_LONG ? (d + CHECK_EVERY) & ~(CHECK_EVERY - 1u)
                                           : (d + CHECK_EVERY_LONG) & ~(CHECK_EVERY_LONG - 1u);
        return t0 + min(nd, t_end - t0);
    };
    uint32_t t_chk = next_check();
    /* a word that stays 0: what a lane without a port reads as its arrival,
     * and where it writes its (empty) departure */
    LDSP uint32_t *const zero = fw + S;
    /* every wavefront holds hosts only or switch ports only */
    const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
    const bool w_host = wv * 64u < SB, w_sw = !w_host && wv * 64u < nt;
    /* with every delay 1, the staging words this lane reads and writes at
     * ticks of parity 0 and 1 */
    const bool port = pr.flags & PF_USED;                      /* slots of absent hosts and gaps have none */
    LDSP uint32_t *const rd1[2] = {port ? sdesc + pr.stg : zero, port ? sdesc + NS + pr.stg : zero};
    LDSP uint32_t *const wr1[2] = {port ? sdesc + NS + pr.pstg : zero, port ? sdesc + pr.pstg : zero};

    /* One tick t.  P is t & 1 when the caller knows it at compile time (every
     * delay 1: staging has two slots, so the addresses of a tick of either
     * parity are loop constants), else P is 2 and both come from t. */
    /* KC: the kind of this wavefront (1 hosts, 2 switch ports, 0 none); each
     * kind runs its own copy of the loop, so values live in one kind's
     * registers never have to be merged with another's */
    auto tick = [&](auto KC, auto PC) -> bool {
        constexpr uint32_t KK = decltype(KC)::value;
        constexpr uint32_t PK = decltype(PC)::value;
        const uint32_t P = PK < 2 ? PK : (t & 1u);
        LDSP uint32_t *rdp, *wrp;                               /* staging: this tick's arrival, departure */
        if constexpr (PK < 2) {
            rdp = rd1[PK];
            wrp = wr1[PK];
        } else {
            uint32_t dst = sb + doff;
            if (dst >= wsz) dst -= wsz;
            rdp = port ? sdesc + sb + pr.stg : zero;
            wrp = port ? sdesc + dst + pr.pstg : zero;
        }
        LDSP uint32_t *fw_prev = fw + (P ^ 1u) * FWS;           /* what the outputs took at t - 1 */
        LDSP uint32_t *fw_cur = fw + P * FWS;                   /* ... take at t */
        if constexpr (KK == 2) {
            /* ---- round 1: the arriving packet; what the outputs took from
             * this buffer and from the one it feeds during t - 1 */
            const uint32_t e = *rdp;
            const uint32_t w = fw_prev[pool];
            const uint32_t pw = fw_prev[peer_pool];
            fw_cur[pool] = 0u;
            mask |= w & 0xFFFFu;
            ne &= ~(w >> 16);
            seen += (uint32_t)__builtin_popcount((uint32_t)(uint16_t)pw);
            /* arrival: append to the queue toward the egress the descriptor names */
            if (e != 0) {
                const uint32_t o = e & 7u;
                fmin = min(fmin, mask);                           /* 0: a packet met a full buffer */
                const uint32_t s = (uint32_t)__builtin_ctz(mask | 0x8000u);   /* in range even when mask is 0 */
                mask &= mask - 1;
                /* drop this switch's hop: the bits shifted into the top of the
                 * route field are never read, since a path has at most
                 * RING_MAX_HOPS switches */
                *(LDSP uint32_t *)(pd_me + __umul24(s, S4)) = ((e >> 3) & RD_ROUTE_MASK) | (e & ~RD_ROUTE_MASK);
                pn_me[__umul24(s, S)] = (uint8_t)Q_EMPTY;
                const uint32_t o4 = o * 4u;
                /* link behind the queue's tail, or make it the head; the
                 * output's non-empty bit is already set when the queue holds
                 * packets, so setting it again changes nothing */
                const uint32_t tl = __builtin_amdgcn_ubfe(tails, o4, 4);
                LDSP uint8_t *lnk = __builtin_amdgcn_ubfe(ne, o, 1) ? pn_me + __umul24(tl, S) : head + hb0 + 8 * o;
                *lnk = (uint8_t)s;
                __hip_atomic_fetch_or(nzw + pr.row + o, 1u << local, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                tails += (s - tl) << o4;                          /* the tail nibble becomes s */
                ne |= 1u << o;
            }
            wave_lds_fence();
            /* ---- round 2: forwarding.  Candidates: the inputs whose queue
             * toward this output holds a packet; the grant goes to the first
             * from rr; credit is the far buffer's room as of the end of t - 1 */
            uint32_t nz = nzw[row];
            uint64_t hrow = *(const LDSP uint64_t *)(head + row * 8u);
            pin(nz); pin(hrow);
            uint32_t out = 0;
            const bool go = nz != 0 && pushed - seen < qcap;
            if constexpr (PK < 2) {
                /* every delay is 1: the wavefront's latest send (the two lane
                 * masks the comparisons already produce) */
                if ((__ballot(nz != 0) & __ballot(pushed - seen < qcap)) != 0ull) last_w = t + 1;
            }
            if (go) {
                /* nz != 0; bits at or above deg are 0, so a search from
                 * rr == deg wraps to input 0 */
                const uint32_t i = (rr + (uint32_t)__builtin_ctz(__builtin_amdgcn_alignbit(nz, nz, rr))) & 7u;
                const uint32_t s = (uint32_t)(hrow >> (8 * i)) & 0xFFu;
                const uint32_t qa = __umul24(s, S) + pool0 + i;
                /* ---- round 3: the packet and its successor in the queue */
                const uint32_t d = pdesc[qa];
                const uint32_t nx = pnxt[qa];
                head[row * 8u + i] = (uint8_t)nx;
                /* 1 when the queue is now empty: slots are below 16, Q_EMPTY is 0xFF */
                const uint32_t em = nx >> 7;
                __hip_atomic_fetch_or(fw_cur + pool0 + i, (1u << s) | (em << (16 + local)),
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                nzw[row] = nz & ~(em << i);
                out = d;
                pushed++;
                if constexpr (PK == 2) last_tx1 = t + 1;
                rr = i + 1;
            }
            *wrp = out;
        } else if constexpr (KK == 1) {
            /* ---- round 1: the arriving packet, the far buffer's pops, and
             * the first ready pair from rr */
            const uint32_t e = *rdp;
            const uint32_t pw = fw_prev[peer_pool];
            seen += (uint32_t)__builtin_popcount(pw & 0xFFFFu);
            const bool any = mask != 0;
            const uint32_t j = any ? (rr + (uint32_t)__builtin_ctz(__builtin_amdgcn_alignbit(mask, mask, rr))) & 31u : 0u;
            const RPair pj = rpair_load(pair_me + __umul24(j, SB));
            if (e != 0) delivered++;
            /* ---- round 2, when a flow's last packet arrives: its pair and
             * ring channel */
            const uint32_t k = (e >> RD_PAIR_SHIFT) & 31u;
            const bool last = e & RD_LAST;
            uint32_t k_snd = 0, k_rcv = 0;
            bool woke = false;
            if (last) {
                const RPair pk = rpair_load(pair_me + __umul24(k, SB));
                const RGrp gk = rgrp_load(grp + ((e >> RD_GRP_SHIFT) & 1023u));
                /* the flow is received: RD = t */
                const uint32_t ri = GI_PRED(pk.gi), rpos = pk.rcv;
                const uint32_t fid = rfid(gk, ri, rpos);
                dq[qn] = ((uint64_t)fid << 32) | t;
                qn++;
                tmax = t;
                left--;
                if (rpos >= gk.RS) fault = 1;                     /* a flow no one sends */
                if (rec) rec[fid] = t;
                k_rcv = rpos + 1u;
                pair_me[__umul24(k, SB)].rcv = k_rcv;
                /* the partner's next send waits on this receive (it is idle
                 * only at a step > 0 of a round: step 0 waits on nothing but
                 * its own last send) */
                k_snd = pk.snd;
                const uint32_t spos = RP_POS(k_snd);
                if (RP_ST(k_snd) == CS_IDLE && k_rcv >= spos) {
                    const uint32_t i = GI_RANK(pk.gi);
                    k_snd = (CS_ACTIVE << 30) | (spos << 16) | rsize(gk, i + 2u * gk.N, spos);
                    mask |= 1u << k;
                    last_act1 = t + 1;
                    if (rec) rec[n_flows + rfid(gk, i, spos)] = t;
                    pair_me[__umul24(k, SB)].snd = k_snd;
                    woke = true;
                }
            }
            /* ---- the NIC: one packet of the first ready pair from rr, while
             * the far buffer has room.  That pair is j, read in round 1,
             * unless a pair woken above comes first; pair k's record was
             * rewritten above, so its values come from registers. */
            uint32_t out = 0;
            if (mask != 0 && pushed - seen < qcap) {
                const bool kfirst = woke && (!any || ((k - rr) & 31u) < ((j - rr) & 31u));
                const uint32_t c = kfirst ? k : j;
                const bool usek = last && c == k;
                uint32_t snd = usek ? k_snd : pj.snd;
                const uint32_t gi = usek ? pair_me[__umul24(k, SB)].gi : pj.gi;
                out = (usek ? pair_me[__umul24(k, SB)].desc : pj.desc) | (RP_REM(snd) == 1u ? RD_LAST : 0u);
                pushed++;
                last_tx1 = t + 1;
                rr = c + 1u;   /* 32 rotates as 0; c + 1 == n_out wraps over empty bits */
                if (RP_REM(snd) == 1u) {
                    /* the flow's last packet leaves: SD = t + 1 */
                    const uint32_t rpos = usek ? k_rcv : pj.rcv;
                    const RGrp g = rgrp_load(grp + GI_GRP(gi));
                    const uint32_t spos = RP_POS(snd), np = spos + 1u;
                    mask &= ~(1u << c);
                    if (rec) rec[2 * n_flows + rfid(g, GI_RANK(gi), spos)] = t + 1;
                    if (np >= g.RS) {
                        snd = (CS_DONE << 30) | (np << 16);
                    } else {
                        /* the next flow starts at t + 1 if its receive
                         * predecessor (the partner's flow np - 1) is in, or
                         * if it opens a round; otherwise it waits for it */
                        const uint32_t step = np - __umul24(__umulhi(np << 8, g.mS), g.S);
                        if (step == 0 || rpos >= np) {
                            snd = (CS_ACTIVE << 30) | (np << 16) | rsize(g, GI_RANK(gi) + 2u * g.N, np);
                            mask |= 1u << c;
                            last_act1 = t + 2;
                            if (rec) rec[n_flows + rfid(g, GI_RANK(gi), np)] = t + 1;
                        } else {
                            snd = (CS_IDLE << 30) | (np << 16);
                        }
                    }
                } else {
                    snd -= 1u;
                }
                pair_me[__umul24(c, SB)].snd = snd;
            }
            *wrp = out;
            if (__ballot(qn == RING_DQ) != 0ull) flush_digest();
        }
        t++;
        if constexpr (PK == 2) {
            sb += NS;
            if (sb == wsz) sb = 0;
        }
        if (t == t_chk) {
            last_tx1 = max(last_tx1, last_w);
            const uint32_t max_arr = last_tx1 ? last_tx1 - 1 + pr.delay : 0;
            const uint32_t anyl = __ballot(left > 0) != 0ull;
            const uint32_t ts = wave_max_u32(max(max(last_tx1, last_act1), max_arr));
            /* one slot per wavefront and parity, rewritten by every check of
             * that parity; the reads of a check end before the next check's
             * barrier, so the next write to the same parity cannot race them */
            if (lane == 0) { sh.chk_any[par][wave] = anyl; sh.chk_max[par][wave] = ts; }
            __syncthreads();
            uint32_t anyw = 0, tsw = hist;
            for (uint32_t w = 0; w < nwaves; w++) { anyw |= sh.chk_any[par][w]; tsw = max(tsw, sh.chk_max[par][w]); }
            par ^= 1;
            if (!anyw) { done = true; return true; }
            if (tsw <= t - 1) { dead = true; t_dead = tsw; return true; }
            if (t >= t_end) return true;
            t_chk = next_check();
        } else {
            __syncthreads();
        }
        return false;
    };
    auto loop = [&](auto KC) {
        if (W == 2) {
            /* every delay is 1: ticks in pairs, even then odd */
            bool stop = t >= t_end;
            if (!stop && (t & 1u)) stop = tick(KC, std::integral_constant<uint32_t, 1>());
            while (!stop) {
                if (tick(KC, std::integral_constant<uint32_t, 0>())) break;
                stop = tick(KC, std::integral_constant<uint32_t, 1>());
            }
        } else {
            while (t < t_end)
                if (tick(KC, std::integral_constant<uint32_t, 2>())) break;
        }
    };
    /* every wavefront passes the same barriers: the loops differ only in
     * what a tick does between them */
    if (w_host) loop(std::integral_constant<uint32_t, 1>());
    else if (w_sw) loop(std::integral_constant<uint32_t, 2>());
    else loop(std::integral_constant<uint32_t, 0>());

    if (w_host) flush_digest();
    last_tx1 = max(last_tx1, last_w);
    const uint32_t max_arr = last_tx1 ? last_tx1 - 1 + pr.delay : 0;
    if (fmin == 0) fault = 1;
    {
        const uint4 *src = (const uint4 *)(lds + rw_off);
        uint4 *dst = (uint4 *)(arena_g + rw_off);
        for (uint32_t i = tid; i < (lds_bytes - rw_off) / 16; i += nth) dst[i] = src[i];
    }
    if (used) {
        pv.pushed = pushed; pv.rr = rr; pv.mask = mask; pv.ne = ne; pv.seen = seen;
        pv.tails = is_host ? left : tails;
        ((RingPriv *)(arena_g + H->o_priv))[tid] = pv;
    }
    uint64_t s0 = wave_sum_u64(pushed - pushed0), s1 = wave_sum_u64(delivered), s2 = wave_sum_u64(digest);
    uint32_t m0 = wave_max_u32(tmax), m1 = wave_max_u32(last_tx1), m2 = wave_max_u32(last_act1),
             m3 = wave_max_u32(max_arr), m4 = wave_max_u32(fault);
    if (lane == 0) {
        sh.sum[0][wave] = s0; sh.sum[1][wave] = s1; sh.sum[2][wave] = s2;
        sh.mx[0][wave] = m0; sh.mx[1][wave] = m1; sh.mx[2][wave] = m2; sh.mx[3][wave] = m3; sh.mx[4][wave] = m4;
    }
    __syncthreads();
    if (tid == 0) finish_state(stp, sh, nwaves, t, done, dead, t_dead);
    __syncthreads();
}

/* Kernel kinds: the general path (plain, with tasks, with congestion control),
 * and the compact path for 8- or 16-byte queue rows and 16- or 32-bit packet
 * descriptors, two of them also with trees, send/recv groups and gated rings.
 * Each kind is its own kernel so that each gets its own register allocation. */
/* The placement of a general-path arena: all of it in LDS if it fits; else
 * its switch and NIC state if that fits; else its port table if that fits;
 * else nothing. */
__device__ __forceinline__ int place_of(const KParams &kp, const ArenaHdr *H)
{
    if (H->bytes <= kp.lds_bytes) return PL_LDS;
    if (kp.lds_bytes && H->ro_hot + (H->rw_hot - H->rw_off) <= kp.lds_bytes) return PL_SPLIT;
    const uint32_t port_b = (H->n_ports * (uint32_t)sizeof(PortRO) + 15u) & ~15u;
    if (kp.lds_bytes && port_b <= kp.lds_bytes) return PL_PORTS;
    return PL_HBM;
}

template <int KIND>
__device__ __forceinline__ void run_one(const KParams &kp, uint32_t x, uint8_t *arena, uint8_t *lds, Shared &sh)
{
    if constexpr (KIND == 0 || KIND == KIND_GENERAL_TASKS || KIND == KIND_GENERAL_CC || KIND == KIND_GENERAL_SPRAY) {
        constexpr bool T = KIND != 0, CC = KIND == KIND_GENERAL_CC, SP = KIND == KIND_GENERAL_SPRAY;
        /* every placement is its own inlined copy of the tick loop */
        switch (place_of(kp, (const ArenaHdr *)arena)) {
        case PL_LDS: run_experiment<PL_LDS, T, CC, SP>(kp, x, arena, lds, sh); break;
        case PL_SPLIT: run_experiment<PL_SPLIT, T, CC, SP>(kp, x, arena, lds, sh); break;
        case PL_PORTS: run_experiment<PL_PORTS, T, CC, SP>(kp, x, arena, lds, sh); break;
        default: run_experiment<PL_HBM, T, CC, SP>(kp, x, arena, lds, sh); break;
        }
    } else if constexpr (KIND == KIND_RING) {
        run_ring(kp, x, arena, lds, sh);
    } else if constexpr (KIND == KIND_COMPACT_X8) {
        run_compact<1, uint16_t, true, true>(kp, x, arena, lds, sh);
    } else if constexpr (KIND == KIND_COMPACT_X16) {
        run_compact<2, uint16_t, false, true>(kp, x, arena, lds, sh);
    } else {
        /* compact kinds: 1 + (16-byte rows << 2 | 32-bit descriptors << 1 | some link faster than 1) */
        constexpr int c = KIND - 1;
        run_compact<(c & 4) ? 2 : 1, typename std::conditional<(c & 2) != 0, uint32_t, uint16_t>::type, (c & 1) == 0,
                    false>(kp, x, arena, lds, sh);
    }
}

/* Persistent loop: each workgroup claims the next experiment of its kind (the
 * order array lists the biggest experiments first) until none are left. */
template <int KIND>
__device__ __forceinline__ void megakernel_body(const KParams &kp)
{
    extern __shared__ __align__(16) uint8_t lds_dyn[];
    __shared__ Shared sh;
    const uint64_t *arena_off = (const uint64_t *)(kp.ws + kp.o_arena_off);
    const uint32_t *order = (const uint32_t *)(kp.ws + kp.o_order) + kp.order_base;
    const ExpState *states = (const ExpState *)(kp.ws + kp.o_state);
    for (;;) {
        if (threadIdx.x == 0) sh.exp = atomicAdd(kp.claim, 1u);
        __syncthreads();
        /* the same for every lane: saying so keeps everything derived from it
         * (arena, header fields, per-experiment flags) in scalar registers */
        const uint32_t e = __builtin_amdgcn_readfirstlane(sh.exp);
        __syncthreads();
        if (e >= kp.n_run) break;
        const uint32_t x = order[e];
        if (states[x].status != 1) continue;
        run_one<KIND>(kp, x, kp.ws + arena_off[x], lds_dyn, sh);
    }
}

extern "C" __global__ void __launch_bounds__(1024) msim_megakernel(KParams kp) { megakernel_body<0>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c8h_r1(KParams kp) { megakernel_body<1>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c8h(KParams kp) { megakernel_body<2>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c8w_r1(KParams kp) { megakernel_body<3>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c8w(KParams kp) { megakernel_body<4>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c16h_r1(KParams kp) { megakernel_body<5>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c16h(KParams kp) { megakernel_body<6>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c16w_r1(KParams kp) { megakernel_body<7>(kp); }
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_c16w(KParams kp) { megakernel_body<8>(kp); }
/* at most 512 threads: the task code needs more than 128 registers per lane */
extern "C" __global__ void __launch_bounds__(512) msim_megakernel_t(KParams kp) { megakernel_body<KIND_GENERAL_TASKS>(kp); }
/* the general path with congestion control (and a task graph if the experiment has one) */
extern "C" __global__ void __launch_bounds__(512) msim_megakernel_cc(KParams kp) { megakernel_body<KIND_GENERAL_CC>(kp); }
/* compact kinds that also carry trees, send/recv groups and gated rings; their
 * extra rules need registers that 1024-thread kernels do not have */
extern "C" __global__ void __launch_bounds__(768) msim_megakernel_c8h_r1_x(KParams kp) { megakernel_body<KIND_COMPACT_X8>(kp); }
extern "C" __global__ void __launch_bounds__(768) msim_megakernel_c16h_x(KParams kp) { megakernel_body<KIND_COMPACT_X16>(kp); }
/* the general path with packet spraying (and a task graph if the experiment has one) */
extern "C" __global__ void __launch_bounds__(512) msim_megakernel_sp(KParams kp) { megakernel_body<KIND_GENERAL_SPRAY>(kp); }
/* rings only at rate 1 on switches of at most 8 ports (the ring format) */
extern "C" __global__ void __launch_bounds__(1024) msim_megakernel_ring(KParams kp) { megakernel_body<KIND_RING>(kp); }

static const void *kernel_of(uint32_t kind)
{
    switch (kind) {
    case 0: return (const void *)msim_megakernel;
    case 1: return (const void *)msim_megakernel_c8h_r1;
    case 2: return (const void *)msim_megakernel_c8h;
    case 3: return (const void *)msim_megakernel_c8w_r1;
    case 4: return (const void *)msim_megakernel_c8w;
    case 5: return (const void *)msim_megakernel_c16h_r1;
    case 6: return (const void *)msim_megakernel_c16h;
    case 7: return (const void *)msim_megakernel_c16w_r1;
    case 8: return (const void *)msim_megakernel_c16w;
    case KIND_GENERAL_TASKS: return (const void *)msim_megakernel_t;
    case KIND_GENERAL_CC: return (const void *)msim_megakernel_cc;
    case KIND_COMPACT_X8: return (const void *)msim_megakernel_c8h_r1_x;
    case KIND_COMPACT_X16: return (const void *)msim_megakernel_c16h_x;
    case KIND_RING: return (const void *)msim_megakernel_ring;
    default: return (const void *)msim_megakernel_sp;
    }
}

/* Prepares launches: zeroes their experiment queue counters (a kernel, not a
 * memset, so that a captured graph replays it faithfully). */
extern "C" __global__ void msim_prepare(uint32_t *words, uint32_t n)
{
    if (blockIdx.x == 0 && threadIdx.x < n) words[threadIdx.x] = 0;
}

/* Experiment queue counters of msim_run_noalloc: MSIM_SCRATCH_WORDS words per
 * GPU, held until the process ends.  Host code never passes this name to a
 * kernel: it passes the device address msim_scratch_words() looked up. */
static __device__ __align__(256) uint32_t scratch[MSIM_SCRATCH_WORDS];

/* Restores every experiment to tick 0: copies the pristine mutable part back
 * into each arena, resets progress and clears recorded per-flow ticks. */
extern "C" __global__ void msim_reset_kernel(KParams kp, uint64_t o_rec_all, uint64_t rec_words)
{
    const uint64_t *arena_off = (const uint64_t *)(kp.ws + kp.o_arena_off);
    const uint64_t *prist = (const uint64_t *)(kp.ws + kp.o_pristine);
    ExpState *states = (ExpState *)(kp.ws + kp.o_state);
    for (uint32_t x = blockIdx.x; x < kp.n_exp; x += gridDim.x) {
        uint8_t *arena = kp.ws + arena_off[x];
        const uint32_t bytes = ((const ArenaHdr *)arena)->bytes;
        const uint32_t rw = ((const ArenaHdr *)arena)->rw_off;
        const uint4 *src = (const uint4 *)(kp.ws + prist[x]);
        uint4 *dst = (uint4 *)(arena + rw);
        for (uint32_t i = threadIdx.x; i < (bytes - rw) / 16; i += blockDim.x) dst[i] = src[i];
        if (threadIdx.x == 0) {
            ExpState s = {};
            const ArenaHdr *ah = (const ArenaHdr *)arena;
            s.status = ah->n_flows == 0 && (ah->mode != MODE_GENERAL || ah->n_task == 0) ? 0u : 1u;
            states[x] = s;
        }
    }
    uint32_t *rec = (uint32_t *)(kp.ws + o_rec_all);
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rec_words;
         i += (uint64_t)gridDim.x * blockDim.x)
        rec[i] = 0xFFFFFFFFu;
}

/* --------------------------------------------------------- host launchers */

/* Device address of `scratch` on the current device, looked up once per
 * device with that device current. */
extern "C" hipError_t msim_scratch_words(uint32_t **out)
{
    static std::mutex mu;
    static uint32_t *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = (uint32_t *)p;
    }
    *out = addr[dev];
    return hipSuccess;
}

/* Zeroes n_clear (<= 64) queue counters at clear if n_clear > 0, then launches a kernel kind. */
extern "C" hipError_t msim_launch_run(const KParams *kp, uint32_t kind, uint32_t grid, uint32_t block,
                                      uint32_t lds, uint32_t *clear, uint32_t n_clear, hipStream_t stream)
{
    if (n_clear) {
        if (n_clear > 64) return hipErrorInvalidValue;
        hipLaunchKernelGGL(msim_prepare, dim3(1), dim3(64), 0, stream, clear, n_clear);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    void *args[] = {(void *)kp};
    return hipLaunchKernel(kernel_of(kind), dim3(grid), dim3(block), args, lds, stream);
}

extern "C" hipError_t msim_launch_reset(const KParams *kp, uint64_t o_rec_all, uint64_t rec_words,
                                        hipStream_t stream)
{
    uint32_t grid = kp->n_exp < 4096 ? kp->n_exp : 4096;
    hipLaunchKernelGGL(msim_reset_kernel, dim3(grid), dim3(256), 0, stream, *kp, o_rec_all, rec_words);
    return hipGetLastError();
}

extern "C" hipError_t msim_occupancy(uint32_t kind, uint32_t block, uint32_t lds, int *blocks_per_cu)
{
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, kernel_of(kind), (int)block, lds);
}

extern "C" hipError_t msim_set_lds_limit(uint32_t kind, uint32_t lds)
{
    return hipFuncSetAttribute(kernel_of(kind), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}
