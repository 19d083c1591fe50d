/*
 * oracle.c -- plain, slow CPU reference of the batched packet simulator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load
 * this file; only the test-suite, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or helper with the HIP
 * library: the two read the same generator arrays and compute everything else
 * on their own.
 *
 * What it computes (one experiment at a time, tick by tick):
 *   Multiverse ("Accelerating Design Space Exploration for LLM Training Systems
 *   with Multi-experiment Parallel Simulation"), section 3.2 "System execution
 *   graph": every simulation step runs Schedule -> Send -> NIC send -> Forward ->
 *   Transmit -> NIC receive in a fixed order; section 4.2 "Pull-based data
 *   synchronisation": each ingress keeps a to-do set of egress ports and each
 *   egress pulls from the ingresses; section 5 "Implementation": the step is the
 *   smallest link delay, flows come from NCCL's ring algorithms, ECMP balances
 *   load.  AutoCCL ("Automated Collective Communication Tuning"), section 2.3:
 *   a message is cut into NC channels processed concurrently, and each channel
 *   moves its chunks of size C one after the other.  AlpaComm ("On Optimizing
 *   the Communication of Model Parallelism"), section 3.1, Fig. 3d: a receiver
 *   forwards a partition once it holds all of it.
 *
 * Where the pages leave a step open, the plainest reading is taken; every such
 * reading is one of the numbered tick rules below.
 *
 * Tick rules (integer time; one tick = the smallest link delay):
 *  R1  A message of B bytes is ceil(B / pkt_bytes) packets.
 *  R2  A node's ports are numbered by the order of its cables in the input.
 *      Every host has exactly one cable.  Cables join nodes of different layers.
 *  R3  Every switch ingress port has room for Q packets.  The room counts every
 *      packet sent on the cable into it and not yet forwarded, also packets still
 *      on the wire.  Inside, one FIFO per egress port (virtual output queue) in
 *      sending order.  A packet is eligible once its arrival tick <= t.  Hosts
 *      take every packet.
 *  R4  Routing: at a node, the candidates for destination host h are the alive
 *      ports whose neighbour lies on a shortest up-then-down path to h (moves to
 *      a higher layer, then moves to a lower one), in port order; a connection
 *      picks cand[H mod |cand|] with H = fmix32(key ^ fmix32(node ^ seed)),
 *      fmix32 being MurmurHash3's 32-bit finaliser; key = connection index.
 *  R5  A flow is (connection, size >= 1 packets, predecessors).  A predecessor is
 *      RECV (its last packet has arrived: RD <= t) or SEND (its last packet has
 *      left: SD <= t, SD = tick of the last send + 1).  The flows of a connection
 *      are chained by SEND predecessors.
 *  R6  Phases of tick t:
 *      A  packets with arrival tick t reach their host: the flow's received count
 *         grows; at its size, RD = t.
 *      B  a not yet active flow whose predecessors are all met becomes active
 *         (activation tick t).
 *      C  every output takes credit = Q - occupancy of the ingress it feeds
 *         (occupancy as left by tick t-1; no limit towards a host).
 *      D  rounds m = 0 .. R-1 (R = largest rate).  In round m every alive output
 *         with m < rate and credit > 0 grants the first candidate input found
 *         going round from its pointer rr: at a switch the ingress ports whose
 *         FIFO for this output has an eligible head; at a host its connections
 *         (in connection index order) whose active flow still has packets to
 *         send.  The packet leaves with arrival tick t + delay, credit drops by
 *         one, rr becomes the granted input + 1.  All grants of a round are
 *         decided on the state at the start of the round.  A flow whose last
 *         packet leaves gets SD = t + 1.
 *      E  done once every flow has an RD; completion tick = the largest RD.  A
 *         tick with no sending, no activation and nothing on the wire, while not
 *         done, is a deadlock at that tick.
 *  W1  Ring all-reduce / all-gather over members m_0..m_{N-1} (rank i sends to
 *      rank i+1 mod N): P packets; channel c carries P/NC + [c < P mod NC];
 *      p = chunk_bytes / pkt_bytes; rounds R_c = ceil(P_c / (N p)), the last
 *      one folded into the previous one when it would hold fewer than N packets;
 *      a round of X packets has chunks k of X/N + [k < X mod N] packets.
 *      All-reduce has 2(N-1) steps, all-gather N-1.  At step s rank i sends chunk
 *      (i - s) mod N (all-gather, and the first N-1 all-reduce steps) or
 *      (i + 1 - (s - N + 1)) mod N (the later all-reduce steps) to rank i+1.
 *      Predecessors of flow (c, r, s, i): s >= 1: RECV (c, r, s-1, i-1) and
 *      SEND (c, r, s-1, i); s = 0, r >= 1: SEND (c, r-1, S-1, i).
 *  W2  Pipelined broadcast along h_0 (source), h_1 .. h_A with K partitions of
 *      P/K + [k < P mod K] packets: flow (j, k) runs h_{j-1} -> h_j with
 *      predecessors RECV (j-1, k) for j >= 2 and SEND (j, k-1) for k >= 1.
 *  W3  Explicit flows: one connection and one flow each, no predecessors.
 *  W5  Ring reduce-scatter (one of the collective algorithms Multiverse section 5
 *      lists): the message is the total input; channels,
 *      rounds and chunks as in W1; N-1 steps in which rank i sends chunk
 *      (i - s) mod N, i.e. the first half of the all-reduce.  With a reduction
 *      that costs no time (A7) its traffic equals the all-gather's.
 *  W6  Send/recv unit task (AlpaComm section 3.1, Figure 3a): member 0 sends the
 *      whole message to members 1 .. A in that order, flow j on connection
 *      (m_0 -> m_j) with predecessor SEND (j-1), so that sends are sequential.
 *      A ring may be gated on an earlier send/recv whose receivers are exactly
 *      its members, in order: rank i's step-0 flow of round 0 of every channel
 *      then also waits on RECV of the send/recv's flow i (Figure 3c's global
 *      all-gather after the scatter).
 *  W7  Tree all-reduce (the tree that AutoCCL section 4.1 contrasts with the
 *      ring, cost log2 N against 2(N-1)): members form a binary tree in order (the parent of
 *      i is (i-1)/2, member 0 the root).  Per channel (split as in W1), the
 *      message goes in chunks of p packets, the last one holding the rest.
 *      For chunk k, node i > 0 sends up to its parent once it has received
 *      chunk k from each of its children; the root's children receive chunk k
 *      once the root has it from all its children, and every other node's
 *      children once that node has received it from its parent.  Each
 *      connection sends its chunks in order (SEND on chunk k-1).
 *  W8  Task graph (the System Simulator's compute graph, Multiverse section 3.1;
 *      the Schedule and AnalyticalSys systems of section 3.2): per workload a
 *      list of tasks in topological order, each a computation of D ticks, an
 *      intra-server collective of D = alpha + ceil(bytes / beta) ticks (the
 *      analytical model of section 4.1, parameters given by the input), or one
 *      of the workload's collectives.  A task starts at the first tick by which
 *      every predecessor has finished; a compute or intra-server task finishes
 *      D ticks later (D >= 1), a collective task when its last flow arrives.  A
 *      collective named by a task cannot start before it: the first flow of
 *      each of its connections also waits for the task's start.  Collectives no
 *      task names start at tick 0.  The experiment is done when every flow has
 *      arrived and every task has finished; its completion tick is the latest
 *      RD or task finish.
 *  W9  Congestion control (Multiverse section 3.2: flows carry congestion-control
 *      variables and an ACK system closes each step; section 5 names DCTCP
 *      among the supported algorithms).  Per experiment, none or DCTCP
 *      (Alizadeh et al., SIGCOMM 2010), restated in integer arithmetic:
 *      - ECN: a packet reaching a switch at tick t is marked when the packets
 *        there for the same egress that arrived before t and were not
 *        forwarded before t number at least K; a mark is kept to the end.
 *      - ACK: a packet delivered at t acknowledges itself at its connection's
 *        source at t + L (L: the sum of the path's link delays, i.e. the same
 *        cables backwards); ACKs take no link capacity and never queue.
 *      - Sender, per connection: window cwnd in 1/256 packet (initially W0
 *        packets), alpha in 1/1024 (initially 1), counters of packets sent and
 *        acknowledged.  The NIC may send for a connection only while sent -
 *        acked < floor(cwnd).  The k ACKs (m marked) arriving in one tick are
 *        applied together: acked += k; cwnd += (k - m) * 65536 / cwnd (one
 *        1/cwnd per unmarked ACK, the pre-batch cwnd); then, once acked reaches
 *        the window end, alpha = alpha - alpha/16 + F/16 with F = 1024 *
 *        marked / acknowledged over the window, cwnd = max(1 packet, cwnd *
 *        (1 - alpha/2)) if any was marked, and the next window ends at the
 *        packets sent so far (the first ends at 0).  cwnd is capped at 65535
 *        packets; every division floors.
 *  W9b DCQCN (Zhu et al., SIGCOMM 2015), the other congestion control: the same
 *      ECN marks; the receiver of a marked packet sends a CNP, at most one
 *      per connection every 608 ticks, reaching the source L ticks later; the
 *      sender keeps a rate RC and target RT (1/65536 packet per tick, both
 *      initially one packet per tick) and alpha (1/1024, initially 1).  A CNP:
 *      RT = RC, RC = max(64, RC - RC alpha / 2048), alpha = alpha - alpha/256 +
 *      4, and the timer, byte and stage counters restart.  Every 640 ticks
 *      without a CNP alpha decays by alpha/256; every 640 ticks and every 2560
 *      packets sent a rate-increase event raises the timer or byte stage count
 *      and: below 5 in both, RT stays (fast recovery); above 5 in both, RT +=
 *      160 (min stage - 5) (hyper increase); else RT += 64 (additive); RT is
 *      capped at one packet per tick; then RC = (RT + RC) / 2.  Timer events
 *      due by a tick come before that tick's CNP and sends (alpha's before the
 *      increase on a tie).  Pacing: a packet leaves no earlier than the
 *      connection's next send time, which the send at tick t sets to
 *      max(previous, t - 65535/65536) + 2^32 / RC in 1/65536 tick (a pacer
 *      that may lag its schedule by under one tick).
 *  W9c HPCC (Li et al., SIGCOMM 2019), the third congestion control: every
 *      switch egress a packet leaves through stamps it with in-band telemetry
 *      (the tick, the egress's count of packets sent, its backlog at the start
 *      of the tick as W9 defines it, its rate); the destination echoes it in
 *      the packet's ACK, which reaches the source L ticks later.  Each
 *      connection keeps a window W (1/256 packet; at most and initially
 *      W_init = T packets, T = 2 L the base round trip, i.e. line rate times T),
 *      a reference window Wc, a utilisation U (1/65536) and an increase stage.
 *      ACKs are taken one by one in sequence order.  The first only records
 *      its telemetry.  Each later one estimates, per hop with a tick between
 *      the two samples, u = min(qlen, previous qlen) / (B T) + (packets sent
 *      between the samples) / (B ticks between them), keeps the largest u and
 *      its tick gap tau (at most T), and sets U = ((T - tau) U + tau u) / T.
 *      Then: with U >= eta = 0.95 or the stage at 5, W = Wc eta / U + W_AI
 *      (stage back to 0), else W = Wc + W_AI (stage + 1); W is kept within 1
 *      packet .. W_init, and Wc and the stage change only on the first ACK
 *      of a packet sent after the previous change (once per round trip).
 *      W_AI = W_init (1 - eta) / 16.  The NIC sends only while sent - acked <
 *      floor(W).
 *  W10 Packet spraying (Multiverse section 5 lists it beside ECMP as a load
 *      balancing algorithm).  Per experiment, ECMP (every packet of a
 *      connection on its one route, R4) or spraying: every packet chooses at
 *      every switch among the same equal-cost candidates, keyed by its
 *      connection and its sequence number s (the count of packets the
 *      connection sent before it): key = conn ^ fmix32(s + 1), egress =
 *      cand[fmix32(key ^ fmix32(switch ^ seed)) mod |cand|].  A packet that
 *      has moved down a layer only moves down.  Delivery stays in order per
 *      connection, as a reliable connection's receiver delivers: a packet that
 *      overtook an earlier one waits until the earlier one has arrived, and a
 *      flow is received when all of its packets and all earlier ones of its
 *      connection have arrived.
 *  Numbering: connections and flows follow the input order of collectives, then
 *  explicit flows; a ring numbers its connections by (channel, rank) and its
 *  flows by (channel, round, step, rank); a broadcast by hop, and (hop, part);
 *  a send/recv by receiver; a tree by channel, then its up connections for
 *  nodes 1 .. N-1 and its down connections for nodes 1 .. N-1, and its flows
 *  by (channel, chunk, connection).
 *  Digest = sum over flows of mix64((flow << 32) | RD) mod 2^64, mix64 being
 *  SplitMix64's output function.
 *
 * Pins (tests/test_oracle_pins.py): closed forms for a single flow, NC = 1
 * rings and the pipelined broadcast; four hand traces; conservation, per-flow
 * bounds and route lengths against an independent breadth-first search.
 * (tests/test_oracle_tasks.py): task chains and fork-joins against the ring
 * closed form plus durations, the analytical duration, and the start rule on a
 * random mixed graph.
 * (tests/test_oracle_collectives.py): two hand traces (a tree, a gated global
 * all-gather), closed forms for two-member trees, sequential sends and the
 * send/recv strategies, reduce-scatter equal to all-gather, and the W6/W7
 * predecessor rules rebuilt in the test and checked through activation ticks.
 * (tests/test_oracle_cc.py): three hand traces of W9 (additive increase, a
 * marked window, an incast whose marks cut both windows), the every-ACK-marked
 * closed form 2L(P-1) + L on three fabrics, and the base model reproduced flow
 * by flow when neither windows nor marks can act.
 * (tests/test_oracle_spray.py): the mixer against the published MurmurHash3
 * vectors; single-path fabrics spray exactly like ECMP; a contention-free
 * two-spine fabric whose sprayed arrivals and in-order completions have a
 * closed form given the hash; equal packet-hops on multi-path fabrics.
 * Parity unpinned (the pages fix no value): which of several equal-cost ECMP
 * candidates the hash picks (only validity and length of a route are pinned),
 * the digest mixer (a checksum; per-flow ticks are compared as well), and the
 * DEADLOCK status (no valid input reaches it under up/down routing).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_S_INCOMPLETE 1
#define ORC_S_DEADLOCK 2
#define ORC_E_INVALID (-1)
#define ORC_E_UNROUTABLE (-2)
#define ORC_E_NOMEM (-3)
#define ORC_E_INVARIANT (-4)

#define NONE 0xFFFFFFFFu
#define INF_DIST 0x3FFFFFFF

enum { KIND_RING_AR = 1, KIND_RING_AG = 2, KIND_BCAST = 3, KIND_RING_RS = 4, KIND_TREE = 5, KIND_SENDRECV = 6 };
enum { PRED_RECV = 0, PRED_SEND = 1, PRED_TASK = 2 };
enum { TASK_COMPUTE = 0, TASK_INTRA = 1, TASK_COLL = 2 };
enum { CC_NONE = 0, CC_DCTCP = 1, CC_DCQCN = 2, CC_HPCC = 3 };
#define HP_ETA 62259u           /* 0.95 in 1/65536 */
#define HP_MAX_STAGE 5u
#define HP_N 16u                /* flows expected to share a link, in W_AI */
#define HP_HOPS 8u              /* switches on a path carrying telemetry */
#define QCN_ONE 65536u          /* one packet per tick */
#define QCN_RMIN 64u
#define QCN_T_INC 640u
#define QCN_T_ALPHA 640u
#define QCN_BYTES 2560u         /* packets between byte-counter events */
#define QCN_F 5u
#define QCN_AI 64u
#define QCN_HAI 160u
#define QCN_CNP_GAP 608u
enum { LB_ECMP = 0, LB_SPRAY = 1 };
#define CWND_MAX (65535u << 8)

/* The batch, exactly as the input generator lays it out. */
typedef struct {
    uint32_t n_topo, n_work, n_exp, pad;
    const uint32_t *topo_node_off;
    const uint8_t *node_layer;
    const uint32_t *topo_cable_off;
    const uint32_t *cable_a, *cable_b;
    const uint8_t *cable_rate_ab, *cable_rate_ba, *cable_delay, *cable_alive;
    const uint32_t *work_coll_off;
    const uint8_t *coll_type;
    const uint64_t *coll_bytes;
    const uint32_t *coll_nc, *coll_chunk_bytes, *coll_k, *coll_member_off, *member_host;
    const uint64_t *work_xflow_off;
    const uint32_t *xflow_src, *xflow_dst, *xflow_pkts;
    const uint32_t *exp_topo, *exp_work, *exp_queue_pkts, *exp_ecmp_seed, *exp_pkt_bytes;
    const uint32_t *coll_gate;   /* per collective: earlier send/recv collective of the workload, or NONE */
    /* tasks (may be NULL): per workload a list in topological order */
    const uint32_t *work_task_off;
    const uint8_t *task_type;
    const uint32_t *task_ticks;      /* compute: duration; intra: alpha */
    const uint64_t *task_bytes;      /* intra: bytes */
    const uint32_t *task_beta;       /* intra: bytes per tick */
    const uint32_t *task_coll;       /* collective task: collective index within the workload */
    const uint32_t *task_pred_off;   /* CSR over all tasks */
    const uint32_t *task_pred;       /* task indices within the workload, each below its task */
    /* congestion control (may be NULL: none) */
    const uint8_t *exp_cc;           /* 0 none, 1 DCTCP */
    const uint32_t *exp_ecn_k;       /* marking threshold, packets */
    const uint32_t *exp_cwnd0;       /* initial window, packets */
    const uint8_t *exp_lb;           /* may be NULL: 0 ECMP, 1 packet spraying */
} orc_batch;

typedef struct {
    int32_t status;        /* ORC_OK (done), ORC_S_INCOMPLETE, ORC_S_DEADLOCK */
    uint32_t t_end;        /* completion tick, deadlock tick, or ticks run */
    uint64_t pkt_hops;     /* transmissions on every link, host NICs included */
    uint64_t delivered;    /* packets received by hosts */
    uint64_t digest;
    uint64_t n_flows;
    uint64_t n_conns;
    uint32_t max_occupancy;/* largest switch ingress occupancy seen */
    uint32_t pad;
} orc_result;

/* ------------------------------------------------------------------ mixers */

static uint32_t fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static uint32_t ecmp_hash(uint32_t key, uint32_t node, uint32_t seed)
{
    return fmix32(key ^ fmix32(node ^ seed));
}

/* ------------------------------------------------------------- structures */

typedef struct {
    uint32_t flow;      /* flow id the packet belongs to */
    uint32_t arrive;    /* arrival tick at the next node */
    uint32_t hop;       /* index in the connection's path of the node it reaches */
    uint32_t mark;      /* ECN mark */
    uint32_t seq;       /* packets its connection sent before it */
    /* HPCC telemetry per switch on the path: tick, egress packets sent,
     * egress backlog, egress rate */
    uint32_t int_ts[HP_HOPS], int_tx[HP_HOPS], int_q[HP_HOPS], int_b[HP_HOPS];
} Pkt;

typedef struct {       /* FIFO of packets (ring buffer of fixed capacity) */
    Pkt *buf;
    uint32_t cap, head, count;
} Fifo;

typedef struct {
    uint32_t node;       /* owner */
    uint32_t peer_node;
    uint32_t peer_port;  /* global port index of the far end */
    uint32_t rate;       /* packets/tick leaving through this port */
    uint32_t delay;
    uint32_t alive;
    uint32_t rr;         /* round-robin pointer of the output */
    uint32_t occ;        /* switch ingress: packets sent into it, not yet forwarded */
    int64_t credit;      /* phase C snapshot, consumed during phase D */
    uint32_t granted;    /* phase D decision of the current round (input index or NONE) */
    uint32_t tx;         /* packets sent through this port so far */
    uint32_t bl;         /* switch egress: backlog at the start of the tick (HPCC) */
    Fifo *voq;           /* switch ingress: one FIFO per egress port of the node */
    Fifo wire;           /* host ingress: packets on the way to the host */
} Port;

typedef struct {
    uint32_t conn, size;
    uint32_t npred;
    uint32_t pred[3];
    uint32_t pkind[3];
    uint32_t sent, recvd, active;
    uint32_t act, sd, rd;
} Flow;

typedef struct {
    uint32_t type, dur;         /* kind; duration of a compute or intra-server task */
    uint32_t pred_off, npred;   /* into Exp.task_pred */
    uint32_t left;              /* collective task: flows not yet received */
    uint32_t start, finish;     /* ticks, NONE until known */
} Task;

typedef struct {
    uint32_t src, dst;
    uint32_t flow_off, nflow;   /* its flows, in sending order, in conn_flows */
    uint32_t cur;               /* position of the flow being / next to be sent */
    uint32_t path_off, path_len;/* nodes and egress ports from source host to destination host */
    uint32_t recv_pos;          /* position of the earliest flow not fully received */
    /* congestion control */
    uint32_t lat;               /* sum of the path's link delays */
    uint32_t cwnd, alpha;       /* 1/256 packet, 1/1024 */
    uint32_t sent, acked;       /* packets over the connection */
    uint32_t wend, wa, wm;      /* window end; ACKs and marked ACKs in the window */
    uint32_t *ackq;             /* ACKs on their way back: (tick << 1 | mark), FIFO */
    uint32_t aq_cap, aq_head, aq_n;
    /* DCQCN: rate, target, stage counters, timers, CNP rate limit, pacing */
    uint32_t rc, rt, tcnt, bcnt, bsent, next_inc, next_alpha, last_cnp;
    uint64_t next_fp;           /* next send time, 1/65536 tick */
    /* HPCC: base round trip, windows, utilisation, stage, the packets sent
     * when Wc last changed, additive step, telemetry of the last ACK */
    uint32_t hT, hw, hwc, hU, hstage, hlast, hwai, hhave, nsw;
    uint32_t L_ts[HP_HOPS], L_tx[HP_HOPS], L_q[HP_HOPS];
    uint32_t *ackint;           /* telemetry riding each ACK in ackq: 4 x HP_HOPS words */
    /* packet spraying: arrival flags by sequence number, in-order point */
    uint8_t *got;
    uint32_t pkts, rnext;
} Conn;

typedef struct {
    /* topology */
    uint32_t n_nodes, n_ports;
    const uint8_t *layer;
    uint32_t *port_off;         /* n_nodes + 1 */
    Port *port;
    /* workload */
    uint32_t n_conn, n_flow;
    Conn *conn;
    Flow *flow;
    uint32_t *conn_flows;
    uint32_t *path_node, *path_port; /* egress local port at each path node */
    /* per host: its connections in index order */
    uint32_t *host_conn_off, *host_conn;
    uint32_t Q, seed, R;
    uint32_t cc, ecn_k, cwnd0;
    uint32_t lb;
    int32_t *dist_down, *dist_any;  /* spraying: per destination node, n_nodes entries each */
    /* tasks */
    uint32_t n_task;
    Task *task;
    uint32_t *task_pred;
    uint32_t *flow_task;        /* per flow: the collective task it belongs to, or NONE */
} Exp;

static void fifo_free(Fifo *f) { free(f->buf); f->buf = NULL; }

static int fifo_init(Fifo *f, uint32_t cap)
{
    f->buf = (Pkt *)calloc(cap ? cap : 1, sizeof(Pkt));
    f->cap = cap ? cap : 1;
    f->head = f->count = 0;
    return f->buf ? 0 : -1;
}

static int fifo_push(Fifo *f, Pkt p)
{
    if (f->count == f->cap) {            /* grow: only host wires can need it */
        uint32_t ncap = f->cap * 2;
        Pkt *nb = (Pkt *)malloc(sizeof(Pkt) * ncap);
        if (!nb) return -1;
        for (uint32_t i = 0; i < f->count; i++) nb[i] = f->buf[(f->head + i) % f->cap];
        free(f->buf);
        f->buf = nb; f->cap = ncap; f->head = 0;
    }
    f->buf[(f->head + f->count) % f->cap] = p;
    f->count++;
    return 0;
}

static Pkt *fifo_front(Fifo *f) { return f->count ? &f->buf[f->head] : NULL; }

static Pkt fifo_pop(Fifo *f)
{
    Pkt p = f->buf[f->head];
    f->head = (f->head + 1) % f->cap;
    f->count--;
    return p;
}

static void exp_free(Exp *x)
{
    if (x->port) {
        for (uint32_t p = 0; p < x->n_ports; p++) {
            if (x->port[p].voq) {
                uint32_t n = x->port_off[x->port[p].node + 1] - x->port_off[x->port[p].node];
                for (uint32_t o = 0; o < n; o++) fifo_free(&x->port[p].voq[o]);
                free(x->port[p].voq);
            }
            fifo_free(&x->port[p].wire);
        }
    }
    free(x->port_off); free(x->port); free(x->flow); free(x->conn_flows);
    free(x->path_node); free(x->path_port); free(x->host_conn_off); free(x->host_conn);
    free(x->task); free(x->task_pred); free(x->flow_task);
    if (x->conn) for (uint32_t c = 0; c < x->n_conn; c++) { free(x->conn[c].ackq); free(x->conn[c].ackint); free(x->conn[c].got); }
    free(x->dist_down); free(x->dist_any);
    free(x->conn);
    memset(x, 0, sizeof(*x));
}

static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

/* -------------------------------------------------------------- topology */

static int build_topology(const orc_batch *b, uint32_t e, Exp *x)
{
    uint32_t t = b->exp_topo[e];
    uint32_t n0 = b->topo_node_off[t], n1 = b->topo_node_off[t + 1];
    uint32_t c0 = b->topo_cable_off[t], c1 = b->topo_cable_off[t + 1];
    x->n_nodes = n1 - n0;
    x->layer = b->node_layer + n0;
    x->port_off = (uint32_t *)calloc(x->n_nodes + 1, sizeof(uint32_t));
    if (!x->port_off) return ORC_E_NOMEM;
    /* count ports per node (R2) */
    for (uint32_t c = c0; c < c1; c++) {
        uint32_t a = b->cable_a[c], bb = b->cable_b[c];
        if (a >= x->n_nodes || bb >= x->n_nodes || a == bb) return ORC_E_INVALID;
        if (x->layer[a] == x->layer[bb]) return ORC_E_INVALID;
        if (b->cable_rate_ab[c] < 1 || b->cable_rate_ba[c] < 1 || b->cable_delay[c] < 1) return ORC_E_INVALID;
        x->port_off[a + 1]++;
        x->port_off[bb + 1]++;
    }
    for (uint32_t n = 0; n < x->n_nodes; n++) {
        if (x->layer[n] == 0 && x->port_off[n + 1] != 1) return ORC_E_INVALID;
        x->port_off[n + 1] += x->port_off[n];
    }
    x->n_ports = x->port_off[x->n_nodes];
    x->port = (Port *)calloc(x->n_ports ? x->n_ports : 1, sizeof(Port));
    uint32_t *fill = (uint32_t *)calloc(x->n_nodes, sizeof(uint32_t));
    if (!x->port || !fill) { free(fill); return ORC_E_NOMEM; }
    x->R = 1;
    for (uint32_t c = c0; c < c1; c++) {
        uint32_t a = b->cable_a[c], bb = b->cable_b[c];
        uint32_t pa = x->port_off[a] + fill[a]++;
        uint32_t pb = x->port_off[bb] + fill[bb]++;
        x->port[pa].node = a; x->port[pa].peer_node = bb; x->port[pa].peer_port = pb;
        x->port[pa].rate = b->cable_rate_ab[c];
        x->port[pb].node = bb; x->port[pb].peer_node = a; x->port[pb].peer_port = pa;
        x->port[pb].rate = b->cable_rate_ba[c];
        x->port[pa].delay = x->port[pb].delay = b->cable_delay[c];
        x->port[pa].alive = x->port[pb].alive = b->cable_alive[c] ? 1 : 0;
        if (b->cable_rate_ab[c] > x->R) x->R = b->cable_rate_ab[c];
        if (b->cable_rate_ba[c] > x->R) x->R = b->cable_rate_ba[c];
    }
    free(fill);
    for (uint32_t p = 0; p < x->n_ports; p++) {
        Port *pp = &x->port[p];
        pp->granted = NONE;
        if (x->layer[pp->node] != 0) {
            uint32_t deg = x->port_off[pp->node + 1] - x->port_off[pp->node];
            pp->voq = (Fifo *)calloc(deg, sizeof(Fifo));
            if (!pp->voq) return ORC_E_NOMEM;
            for (uint32_t o = 0; o < deg; o++)
                if (fifo_init(&pp->voq[o], x->Q)) return ORC_E_NOMEM;
        } else {
            if (fifo_init(&pp->wire, 64)) return ORC_E_NOMEM;
        }
    }
    return ORC_OK;
}

/* --------------------------------------------------------------- workload */

static int is_ring(uint32_t kind) { return kind == KIND_RING_AR || kind == KIND_RING_AG || kind == KIND_RING_RS; }

/* Chunk sent by rank i at step s (W1; the reduce-scatter takes the all-reduce's first half, W5). */
static uint32_t ring_chunk(uint32_t kind, uint32_t N, uint32_t i, uint32_t s)
{
    if (kind != KIND_RING_AR || s < N - 1) return (uint32_t)(((int64_t)i - s % N + N) % N);
    uint32_t s2 = s - (N - 1);
    return (uint32_t)(((int64_t)i + 1 - s2 + 2 * (int64_t)N) % N);
}

/* Appends one connection; returns its index. */
static uint32_t add_conn(Exp *x, uint32_t src, uint32_t dst)
{
    Conn *c = &x->conn[x->n_conn];
    memset(c, 0, sizeof(*c));
    c->src = src; c->dst = dst;
    return x->n_conn++;
}

/* Counts connections and flows of the workload (first pass), validating it. */
static int count_workload(const orc_batch *b, uint32_t e, uint64_t *nconn, uint64_t *nflow)
{
    uint32_t w = b->exp_work[e], t = b->exp_topo[e];
    uint32_t nn = b->topo_node_off[t + 1] - b->topo_node_off[t];
    const uint8_t *layer = b->node_layer + b->topo_node_off[t];
    uint64_t pkt = b->exp_pkt_bytes[e];
    if (pkt == 0) return ORC_E_INVALID;
    *nconn = 0; *nflow = 0;
    for (uint32_t ci = b->work_coll_off[w]; ci < b->work_coll_off[w + 1]; ci++) {
        uint32_t m0 = b->coll_member_off[ci], m1 = b->coll_member_off[ci + 1];
        uint32_t N = m1 - m0;
        for (uint32_t m = m0; m < m1; m++) {
            if (b->member_host[m] >= nn || layer[b->member_host[m]] != 0) return ORC_E_INVALID;
            for (uint32_t m2 = m0; m2 < m; m2++)
                if (b->member_host[m2] == b->member_host[m]) return ORC_E_INVALID;
        }
        uint64_t P = ceil_div(b->coll_bytes[ci], pkt);
        uint32_t kind = b->coll_type[ci];
        uint32_t gate = b->coll_gate ? b->coll_gate[ci] : NONE;
        if (gate != NONE) {
            /* W6: the gate is an earlier send/recv of this workload whose receivers are these members */
            uint32_t gi = b->work_coll_off[w] + gate;
            if (!is_ring(kind) || gi >= ci || b->coll_type[gi] != KIND_SENDRECV) return ORC_E_INVALID;
            if (b->coll_member_off[gi + 1] - b->coll_member_off[gi] != N + 1) return ORC_E_INVALID;
            for (uint32_t i = 0; i < N; i++)
                if (b->member_host[b->coll_member_off[gi] + 1 + i] != b->member_host[m0 + i]) return ORC_E_INVALID;
            for (uint32_t cj = b->work_coll_off[w]; cj < ci; cj++)   /* a send/recv gates one collective */
                if (b->coll_gate[cj] == gate) return ORC_E_INVALID;
        }
        if (is_ring(kind) || kind == KIND_TREE) {
            uint32_t NC = b->coll_nc[ci];
            if (N < 2 || NC < 1 || b->coll_chunk_bytes[ci] == 0 || b->coll_chunk_bytes[ci] % pkt) return ORC_E_INVALID;
            uint64_t p = b->coll_chunk_bytes[ci] / pkt;
            if (kind == KIND_TREE) {
                for (uint32_t c = 0; c < NC; c++) {
                    uint64_t Pc = P / NC + (c < P % NC);
                    if (Pc < 1) return ORC_E_INVALID;
                    *nflow += ceil_div(Pc, p) * 2 * (N - 1);
                    *nconn += 2 * (N - 1);
                }
                continue;
            }
            uint64_t S = kind == KIND_RING_AR ? 2ull * (N - 1) : (uint64_t)(N - 1);
            for (uint32_t c = 0; c < NC; c++) {
                uint64_t Pc = P / NC + (c < P % NC);
                if (Pc < N) return ORC_E_INVALID;
                uint64_t R = ceil_div(Pc, (uint64_t)N * p);
                if (R > 1 && Pc - (R - 1) * N * p < N) R--;
                *nflow += R * S * N;
                *nconn += N;
            }
        } else if (kind == KIND_BCAST) {
            uint64_t K = b->coll_k[ci];
            if (N < 2 || K < 1 || K > P) return ORC_E_INVALID;
            *nconn += N - 1;
            *nflow += (uint64_t)(N - 1) * K;
        } else if (kind == KIND_SENDRECV) {
            if (N < 2 || P < 1 || P >= NONE) return ORC_E_INVALID;
            *nconn += N - 1;
            *nflow += N - 1;
        } else {
            return ORC_E_INVALID;
        }
    }
    for (uint64_t xi = b->work_xflow_off[w]; xi < b->work_xflow_off[w + 1]; xi++) {
        uint32_t s = b->xflow_src[xi], d = b->xflow_dst[xi];
        if (s >= nn || d >= nn || s == d || layer[s] != 0 || layer[d] != 0 || b->xflow_pkts[xi] == 0)
            return ORC_E_INVALID;
        *nconn += 1; *nflow += 1;
    }
    if (b->work_task_off) {
        /* tasks: durations of at least one tick; a collective task names a
         * collective of this workload that no other task names; predecessors
         * come earlier in the list */
        uint32_t t0 = b->work_task_off[w], t1 = b->work_task_off[w + 1];
        uint32_t ncoll = b->work_coll_off[w + 1] - b->work_coll_off[w];
        for (uint32_t k = t0; k < t1; k++) {
            uint32_t ty = b->task_type[k];
            if (ty == TASK_COMPUTE) {
                if (b->task_ticks[k] < 1) return ORC_E_INVALID;
            } else if (ty == TASK_INTRA) {
                if (b->task_beta[k] < 1) return ORC_E_INVALID;
                uint64_t d = (uint64_t)b->task_ticks[k] + ceil_div(b->task_bytes[k], b->task_beta[k]);
                if (d < 1 || d >= NONE) return ORC_E_INVALID;
            } else if (ty == TASK_COLL) {
                if (b->task_coll[k] >= ncoll) return ORC_E_INVALID;
                for (uint32_t j = t0; j < k; j++)
                    if (b->task_type[j] == TASK_COLL && b->task_coll[j] == b->task_coll[k]) return ORC_E_INVALID;
            } else {
                return ORC_E_INVALID;
            }
            for (uint32_t q = b->task_pred_off[k]; q < b->task_pred_off[k + 1]; q++)
                if (b->task_pred[q] >= k - t0) return ORC_E_INVALID;
        }
    }
    if (*nflow >= NONE || *nconn >= NONE) return ORC_E_INVALID;
    return ORC_OK;
}

static void set_flow(Exp *x, uint32_t f, uint32_t conn, uint32_t size)
{
    Flow *fl = &x->flow[f];
    memset(fl, 0, sizeof(*fl));
    fl->conn = conn; fl->size = size;
    fl->act = fl->sd = fl->rd = NONE;
}

static void add_pred(Exp *x, uint32_t f, uint32_t g, uint32_t kind)
{
    Flow *fl = &x->flow[f];
    fl->pred[fl->npred] = g;
    fl->pkind[fl->npred] = kind;
    fl->npred++;
}

/* Tasks of workload w (the task schedule of the System Simulator, Multiverse
 * section 3.1; Schedule and AnalyticalSys of section 3.2).  A collective
 * task's collective cannot start before the task: the first flow of each of
 * its connections gets the task as one more predecessor. */
static int build_tasks(const orc_batch *b, uint32_t w, Exp *x, const uint32_t *coll_f0, const uint32_t *coll_c0)
{
    x->flow_task = (uint32_t *)malloc(sizeof(uint32_t) * (x->n_flow ? x->n_flow : 1));
    if (!x->flow_task) return ORC_E_NOMEM;
    for (uint32_t f = 0; f < x->n_flow; f++) x->flow_task[f] = NONE;
    if (!b->work_task_off) return ORC_OK;
    uint32_t t0 = b->work_task_off[w], t1 = b->work_task_off[w + 1];
    x->n_task = t1 - t0;
    uint32_t np = b->task_pred_off[t1] - b->task_pred_off[t0];
    x->task = (Task *)calloc(x->n_task ? x->n_task : 1, sizeof(Task));
    x->task_pred = (uint32_t *)calloc(np ? np : 1, sizeof(uint32_t));
    if (!x->task || !x->task_pred) return ORC_E_NOMEM;
    for (uint32_t k = 0; k < x->n_task; k++) {
        Task *tk = &x->task[k];
        uint32_t g = t0 + k;
        tk->type = b->task_type[g];
        tk->start = tk->finish = NONE;
        tk->pred_off = b->task_pred_off[g] - b->task_pred_off[t0];
        tk->npred = b->task_pred_off[g + 1] - b->task_pred_off[g];
        for (uint32_t q = 0; q < tk->npred; q++) x->task_pred[tk->pred_off + q] = b->task_pred[b->task_pred_off[g] + q];
        if (tk->type == TASK_COMPUTE) {
            tk->dur = b->task_ticks[g];
        } else if (tk->type == TASK_INTRA) {
            /* the analytical model of section 4.1: alpha + size / beta, in ticks */
            tk->dur = b->task_ticks[g] + (uint32_t)ceil_div(b->task_bytes[g], b->task_beta[g]);
        } else {
            uint32_t cl = b->task_coll[g];
            tk->left = coll_f0[cl + 1] - coll_f0[cl];
            for (uint32_t f = coll_f0[cl]; f < coll_f0[cl + 1]; f++) x->flow_task[f] = k;
            for (uint32_t c = coll_c0[cl]; c < coll_c0[cl + 1]; c++) {
                Flow *fl = &x->flow[x->conn_flows[x->conn[c].flow_off]];
                fl->pred[fl->npred] = k;
                fl->pkind[fl->npred] = PRED_TASK;
                fl->npred++;
            }
        }
    }
    return ORC_OK;
}

static int build_workload(const orc_batch *b, uint32_t e, Exp *x)
{
    uint64_t nconn, nflow;
    int rc = count_workload(b, e, &nconn, &nflow);
    if (rc) return rc;
    uint32_t w = b->exp_work[e];
    uint64_t pkt = b->exp_pkt_bytes[e];
    x->conn = (Conn *)calloc(nconn ? nconn : 1, sizeof(Conn));
    x->flow = (Flow *)calloc(nflow ? nflow : 1, sizeof(Flow));
    x->conn_flows = (uint32_t *)calloc(nflow ? nflow : 1, sizeof(uint32_t));
    if (!x->conn || !x->flow || !x->conn_flows) return ORC_E_NOMEM;
    x->n_conn = 0;
    uint32_t f = 0;
    uint32_t ncoll = b->work_coll_off[w + 1] - b->work_coll_off[w];
    /* first flow and first connection of each collective (one more entry: the end) */
    uint32_t *coll_f0 = (uint32_t *)calloc(ncoll + 1, sizeof(uint32_t));
    uint32_t *coll_c0 = (uint32_t *)calloc(ncoll + 1, sizeof(uint32_t));
    if (!coll_f0 || !coll_c0) { free(coll_f0); free(coll_c0); return ORC_E_NOMEM; }
    for (uint32_t ci = b->work_coll_off[w]; ci < b->work_coll_off[w + 1]; ci++) {
        const uint32_t *mem = b->member_host + b->coll_member_off[ci];
        uint32_t N = b->coll_member_off[ci + 1] - b->coll_member_off[ci];
        uint64_t P = ceil_div(b->coll_bytes[ci], pkt);
        uint32_t kind = b->coll_type[ci];
        uint32_t gate = b->coll_gate ? b->coll_gate[ci] : NONE;
        coll_f0[ci - b->work_coll_off[w]] = f;
        coll_c0[ci - b->work_coll_off[w]] = x->n_conn;
        if (is_ring(kind)) {
            uint32_t NC = b->coll_nc[ci];
            uint64_t p = b->coll_chunk_bytes[ci] / pkt;
            uint32_t S = kind == KIND_RING_AR ? 2 * (N - 1) : N - 1;
            for (uint32_t c = 0; c < NC; c++) {
                uint64_t Pc = P / NC + (c < P % NC);
                uint64_t R = ceil_div(Pc, (uint64_t)N * p);
                if (R > 1 && Pc - (R - 1) * N * p < N) R--;
                uint32_t conn0 = x->n_conn;
                for (uint32_t i = 0; i < N; i++) add_conn(x, mem[i], mem[(i + 1) % N]);
                uint32_t fbase = f;   /* flow (r, s, i) = fbase + (r*S + s)*N + i */
                for (uint64_t r = 0; r < R; r++) {
                    uint64_t X = (r + 1 < R) ? (uint64_t)N * p : Pc - (R - 1) * N * p;
                    for (uint32_t s = 0; s < S; s++) {
                        for (uint32_t i = 0; i < N; i++) {
                            uint32_t k = ring_chunk(kind, N, i, s);
                            uint32_t size = (uint32_t)(X / N + (k < X % N));
                            set_flow(x, f, conn0 + i, size);
                            if (s >= 1) {
                                uint32_t im1 = (i + N - 1) % N;
                                add_pred(x, f, fbase + (uint32_t)((r * S + s - 1) * N + im1), PRED_RECV);
                                add_pred(x, f, fbase + (uint32_t)((r * S + s - 1) * N + i), PRED_SEND);
                            } else if (r >= 1) {
                                add_pred(x, f, fbase + (uint32_t)(((r - 1) * S + S - 1) * N + i), PRED_SEND);
                            } else if (gate != NONE) {
                                /* W6: rank i starts once its piece from the send/recv has arrived */
                                add_pred(x, f, coll_f0[gate] + i, PRED_RECV);
                            }
                            f++;
                        }
                    }
                }
            }
        } else if (kind == KIND_TREE) {
            /* W7: binary tree in member order (parent of i is (i-1)/2); per chunk,
             * every node reduces up once all its children's pieces arrived, and
             * the result flows back down from the root */
            uint32_t NC = b->coll_nc[ci];
            uint64_t p = b->coll_chunk_bytes[ci] / pkt;
            uint32_t E = 2 * (N - 1);   /* connections per channel: up of node i at i-1, down at N-1+i-1 */
            for (uint32_t c = 0; c < NC; c++) {
                uint64_t Pc = P / NC + (c < P % NC);
                uint64_t R = ceil_div(Pc, p);
                uint32_t conn0 = x->n_conn;
                for (uint32_t i = 1; i < N; i++) add_conn(x, mem[i], mem[(i - 1) / 2]);
                for (uint32_t i = 1; i < N; i++) add_conn(x, mem[(i - 1) / 2], mem[i]);
                uint32_t fbase = f;   /* flow (k, connection j) = fbase + k*E + j */
                for (uint64_t k = 0; k < R; k++) {
                    uint32_t size = (uint32_t)(k + 1 < R ? p : Pc - (R - 1) * p);
                    uint32_t fk = fbase + (uint32_t)(k * E);
                    for (uint32_t j = 0; j < E; j++) {
                        set_flow(x, f, conn0 + j, size);
                        if (j < N - 1) {
                            uint32_t i = j + 1;
                            for (uint32_t ch = 2 * i + 1; ch <= 2 * i + 2 && ch < N; ch++)
                                add_pred(x, f, fk + ch - 1, PRED_RECV);
                        } else {
                            uint32_t i = j - (N - 1) + 1, par = (i - 1) / 2;
                            if (par == 0) {
                                for (uint32_t ch = 1; ch <= 2 && ch < N; ch++) add_pred(x, f, fk + ch - 1, PRED_RECV);
                            } else {
                                add_pred(x, f, fk + (N - 1) + par - 1, PRED_RECV);
                            }
                        }
                        if (k >= 1) add_pred(x, f, fk - E + j, PRED_SEND);
                        f++;
                    }
                }
            }
        } else if (kind == KIND_SENDRECV) {
            /* W6: member 0 sends the whole message to members 1, 2, ... one after another */
            uint32_t conn0 = x->n_conn;
            for (uint32_t j = 1; j < N; j++) add_conn(x, mem[0], mem[j]);
            for (uint32_t j = 0; j + 1 < N; j++) {
                set_flow(x, f, conn0 + j, (uint32_t)P);
                if (j >= 1) add_pred(x, f, f - 1, PRED_SEND);
                f++;
            }
        } else { /* KIND_BCAST */
            uint32_t K = b->coll_k[ci];
            uint32_t A = N - 1;
            uint32_t conn0 = x->n_conn;
            for (uint32_t j = 1; j <= A; j++) add_conn(x, mem[j - 1], mem[j]);
            uint32_t fbase = f;   /* flow (j, k) = fbase + (j-1)*K + k */
            for (uint32_t j = 1; j <= A; j++) {
                for (uint32_t k = 0; k < K; k++) {
                    uint32_t size = (uint32_t)(P / K + (k < P % K));
                    set_flow(x, f, conn0 + j - 1, size);
                    if (j >= 2) add_pred(x, f, fbase + (j - 2) * K + k, PRED_RECV);
                    if (k >= 1) add_pred(x, f, fbase + (j - 1) * K + k - 1, PRED_SEND);
                    f++;
                }
            }
        }
    }
    uint32_t coll_end_conn = x->n_conn;
    for (uint64_t xi = b->work_xflow_off[w]; xi < b->work_xflow_off[w + 1]; xi++) {
        uint32_t c = add_conn(x, b->xflow_src[xi], b->xflow_dst[xi]);
        set_flow(x, f, c, b->xflow_pkts[xi]);
        f++;
    }
    x->n_flow = f;
    /* each connection's flows, in flow-id order (which is their sending order) */
    for (uint32_t i = 0; i < f; i++) x->conn[x->flow[i].conn].nflow++;
    uint32_t acc = 0;
    for (uint32_t c = 0; c < x->n_conn; c++) { x->conn[c].flow_off = acc; acc += x->conn[c].nflow; x->conn[c].nflow = 0; }
    for (uint32_t i = 0; i < f; i++) {
        Conn *c = &x->conn[x->flow[i].conn];
        x->conn_flows[c->flow_off + c->nflow++] = i;
    }
    /* hosts' connections, in connection-index order */
    x->host_conn_off = (uint32_t *)calloc(x->n_nodes + 1, sizeof(uint32_t));
    x->host_conn = (uint32_t *)calloc(x->n_conn ? x->n_conn : 1, sizeof(uint32_t));
    if (!x->host_conn_off || !x->host_conn) return ORC_E_NOMEM;
    for (uint32_t c = 0; c < x->n_conn; c++) x->host_conn_off[x->conn[c].src + 1]++;
    for (uint32_t n = 0; n < x->n_nodes; n++) x->host_conn_off[n + 1] += x->host_conn_off[n];
    uint32_t *fill = (uint32_t *)calloc(x->n_nodes, sizeof(uint32_t));
    if (!fill) return ORC_E_NOMEM;
    for (uint32_t c = 0; c < x->n_conn; c++) {
        uint32_t h = x->conn[c].src;
        x->host_conn[x->host_conn_off[h] + fill[h]++] = c;
    }
    free(fill);
    coll_f0[ncoll] = f - (uint32_t)(b->work_xflow_off[w + 1] - b->work_xflow_off[w]);
    coll_c0[ncoll] = coll_end_conn;
    rc = build_tasks(b, w, x, coll_f0, coll_c0);
    free(coll_f0); free(coll_c0);
    return rc;
}

/* ---------------------------------------------------------------- routing */

/* Shortest down-only distance (down) and shortest up-then-down distance (any)
 * from every node to host dst, over alive cables (R4). */
static void distances(const Exp *x, uint32_t dst, int32_t *down, int32_t *any)
{
    uint32_t maxl = 0;
    for (uint32_t n = 0; n < x->n_nodes; n++) {
        down[n] = INF_DIST; any[n] = INF_DIST;
        if (x->layer[n] > maxl) maxl = x->layer[n];
    }
    down[dst] = 0;
    for (uint32_t L = 1; L <= maxl; L++)
        for (uint32_t n = 0; n < x->n_nodes; n++) {
            if (x->layer[n] != L) continue;
            for (uint32_t p = x->port_off[n]; p < x->port_off[n + 1]; p++) {
                const Port *pp = &x->port[p];
                if (!pp->alive || x->layer[pp->peer_node] >= L) continue;
                if (down[pp->peer_node] + 1 < down[n]) down[n] = down[pp->peer_node] + 1;
            }
        }
    for (int32_t L = (int32_t)maxl; L >= 0; L--)
        for (uint32_t n = 0; n < x->n_nodes; n++) {
            if (x->layer[n] != (uint32_t)L) continue;
            int32_t best = down[n];
            for (uint32_t p = x->port_off[n]; p < x->port_off[n + 1]; p++) {
                const Port *pp = &x->port[p];
                if (!pp->alive || x->layer[pp->peer_node] <= (uint32_t)L) continue;
                if (any[pp->peer_node] + 1 < best) best = any[pp->peer_node] + 1;
            }
            any[n] = best;
        }
}

static int build_routes(Exp *x)
{
    uint32_t maxlen = 0;
    int32_t *down = (int32_t *)malloc(sizeof(int32_t) * x->n_nodes);
    int32_t *any = (int32_t *)malloc(sizeof(int32_t) * x->n_nodes);
    uint32_t *cand = (uint32_t *)malloc(sizeof(uint32_t) * (x->n_ports + 1));
    uint32_t *done_for = (uint32_t *)malloc(sizeof(uint32_t) * x->n_nodes);
    if (!down || !any || !cand || !done_for) { free(down); free(any); free(cand); free(done_for); return ORC_E_NOMEM; }
    /* a shortest up-then-down path has at most 2 * (max layer) links */
    uint32_t maxl = 0;
    for (uint32_t n = 0; n < x->n_nodes; n++) if (x->layer[n] > maxl) maxl = x->layer[n];
    maxlen = 2 * maxl + 1;
    if (x->lb == LB_SPRAY) {
        x->dist_down = (int32_t *)malloc(sizeof(int32_t) * (size_t)x->n_nodes * x->n_nodes);
        x->dist_any = (int32_t *)malloc(sizeof(int32_t) * (size_t)x->n_nodes * x->n_nodes);
        if (!x->dist_down || !x->dist_any) { free(down); free(any); free(cand); free(done_for); return ORC_E_NOMEM; }
    }
    x->path_node = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(x->n_conn ? x->n_conn : 1) * (maxlen + 1));
    x->path_port = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(x->n_conn ? x->n_conn : 1) * (maxlen + 1));
    if (!x->path_node || !x->path_port) { free(down); free(any); free(cand); free(done_for); return ORC_E_NOMEM; }
    int rc = ORC_OK;
    /* group connections by destination so distances are computed once per host */
    for (uint32_t dst = 0; dst < x->n_nodes && rc == ORC_OK; dst++) {
        int used = 0;
        for (uint32_t c = 0; c < x->n_conn; c++) if (x->conn[c].dst == dst) { used = 1; break; }
        if (!used) continue;
        distances(x, dst, down, any);
        if (x->lb == LB_SPRAY) {
            memcpy(x->dist_down + (size_t)dst * x->n_nodes, down, sizeof(int32_t) * x->n_nodes);
            memcpy(x->dist_any + (size_t)dst * x->n_nodes, any, sizeof(int32_t) * x->n_nodes);
        }
        for (uint32_t c = 0; c < x->n_conn && rc == ORC_OK; c++) {
            Conn *cn = &x->conn[c];
            if (cn->dst != dst) continue;
            cn->path_off = c * (maxlen + 1);
            uint32_t node = cn->src, len = 0;
            int going_down = 0;
            while (1) {
                x->path_node[cn->path_off + len] = node;
                if (node == dst) { x->path_port[cn->path_off + len] = NONE; break; }
                int32_t need = going_down ? down[node] : any[node];
                if (need >= INF_DIST || len >= maxlen) { rc = ORC_E_UNROUTABLE; break; }
                uint32_t nc = 0;
                for (uint32_t p = x->port_off[node]; p < x->port_off[node + 1]; p++) {
                    const Port *pp = &x->port[p];
                    uint32_t m = pp->peer_node;
                    if (!pp->alive) continue;
                    if (x->layer[m] < x->layer[node]) {
                        if (down[m] + 1 == need) cand[nc++] = p;
                    } else if (!going_down && x->layer[m] > x->layer[node]) {
                        if (any[m] + 1 == need) cand[nc++] = p;
                    }
                }
                if (nc == 0) { rc = ORC_E_UNROUTABLE; break; }
                uint32_t pick = cand[ecmp_hash(c, node, x->seed) % nc];
                x->path_port[cn->path_off + len] = pick - x->port_off[node];
                cn->lat += x->port[pick].delay;
                uint32_t next = x->port[pick].peer_node;
                if (x->layer[next] < x->layer[node]) going_down = 1;
                node = next;
                len++;
            }
            cn->path_len = len + 1;
        }
    }
    free(down); free(any); free(cand); free(done_for);
    return rc;
}

/* ------------------------------------------------------------- simulation */

typedef struct {
    uint32_t *flow_rd, *flow_act, *flow_sd;  /* optional per-flow outputs */
    uint32_t check;                          /* nonzero: verify invariants each tick */
} orc_opts;

/* W10: the egress local port that a sprayed packet (connection c, sequence
 * number seq) takes at switch node, toward c's destination; down_only once it
 * has moved down a layer.  The candidates are those of the ECMP walk. */
static uint32_t spray_egress(const Exp *x, uint32_t c, uint32_t seq, uint32_t node, int down_only)
{
    const uint32_t dst = x->conn[c].dst;
    const int32_t *down = x->dist_down + (size_t)dst * x->n_nodes;
    const int32_t *any = x->dist_any + (size_t)dst * x->n_nodes;
    const int32_t need = down_only ? down[node] : any[node];
    uint32_t cand[64], nc = 0;
    for (uint32_t p = x->port_off[node]; p < x->port_off[node + 1]; p++) {
        const Port *pp = &x->port[p];
        uint32_t m = pp->peer_node;
        if (!pp->alive) continue;
        if (x->layer[m] < x->layer[node]) {
            if (down[m] + 1 == need) cand[nc++] = p - x->port_off[node];
        } else if (!down_only && x->layer[m] > x->layer[node]) {
            if (any[m] + 1 == need) cand[nc++] = p - x->port_off[node];
        }
    }
    if (nc == 0) return NONE;
    const uint32_t key = c ^ fmix32(seq + 1u);
    return cand[ecmp_hash(key, node, x->seed) % nc];
}

/* Global port index of the ingress port at path position h+1 (the far end of
 * the link leaving path position h). */
static uint32_t out_port(const Exp *x, const Conn *c, uint32_t h)
{
    uint32_t node = x->path_node[c->path_off + h];
    return x->port_off[node] + x->path_port[c->path_off + h];
}

/* Sends packet (flow f, currently at path position hop, ECN mark) out of port
 * op at tick t. */
static int transmit(Exp *x, uint32_t op, const Pkt *from, uint32_t f, uint32_t hop, uint32_t mark, uint32_t seq,
                    uint32_t t, uint64_t *hops, uint32_t *max_arrive, uint32_t *max_occ)
{
    Port *o = &x->port[op];
    Port *in = &x->port[o->peer_port];
    const Conn *c = &x->conn[x->flow[f].conn];
    Pkt p;
    if (from) p = *from;
    else memset(&p, 0, sizeof p);
    o->tx++;
    if (x->cc == CC_HPCC && hop > 0) {
        /* W9c: the switch at path position hop stamps its egress */
        if (hop > HP_HOPS) return ORC_E_INVARIANT;
        p.int_ts[hop - 1] = t;
        p.int_tx[hop - 1] = o->tx;
        p.int_q[hop - 1] = o->bl;
        p.int_b[hop - 1] = o->rate;
    }
    p.flow = f;
    p.arrive = t + o->delay;
    p.hop = hop + 1;
    p.mark = mark;
    p.seq = seq;
    if (p.arrive > *max_arrive) *max_arrive = p.arrive;
    (*hops)++;
    if (x->layer[o->peer_node] == 0) {
        return fifo_push(&in->wire, p) ? ORC_E_NOMEM : ORC_OK;
    }
    uint32_t egress;
    if (x->lb == LB_SPRAY) {
        egress = spray_egress(x, x->flow[f].conn, seq, o->peer_node, x->layer[o->node] > x->layer[o->peer_node]);
        if (egress == NONE) return ORC_E_INVARIANT;    /* the candidate sets keep every packet routable */
    } else {
        egress = x->path_port[c->path_off + p.hop];
    }
    in->occ++;
    if (in->occ > *max_occ) *max_occ = in->occ;
    if (in->occ > x->Q) return ORC_E_INVARIANT;        /* credits make this impossible */
    return fifo_push(&in->voq[egress], p) ? ORC_E_NOMEM : ORC_OK;
}

/* W9: packets for egress o of switch n that arrived before tick t and are
 * still queued: the egress's backlog at the start of t. */
static uint32_t egress_backlog(const Exp *x, uint32_t n, uint32_t o, uint32_t t)
{
    const uint32_t deg = x->port_off[n + 1] - x->port_off[n];
    uint32_t backlog = 0;
    for (uint32_t i = 0; i < deg; i++) {
        const Fifo *q = &x->port[x->port_off[n] + i].voq[o];
        for (uint32_t j = 0; j < q->count; j++)
            if (q->buf[(q->head + j) % q->cap].arrive < t) backlog++;
    }
    return backlog;
}

/* W9 ECN: marks the packets that reach switch ingresses at tick t, against
 * each egress's backlog as it stood before any of them arrived. */
static void ecn_mark(Exp *x, uint32_t t)
{
    for (uint32_t n = 0; n < x->n_nodes; n++) {
        if (x->layer[n] == 0) continue;
        uint32_t deg = x->port_off[n + 1] - x->port_off[n];
        for (uint32_t o = 0; o < deg; o++) {
            if (egress_backlog(x, n, o, t) < x->ecn_k) continue;
            for (uint32_t i = 0; i < deg; i++) {
                Fifo *q = &x->port[x->port_off[n] + i].voq[o];
                for (uint32_t j = 0; j < q->count; j++) {
                    Pkt *k = &q->buf[(q->head + j) % q->cap];
                    if (k->arrive == t) k->mark = 1;
                }
            }
        }
    }
}

/* W9 DCTCP: k ACKs, m of them marked, reach connection c's source together. */
static void dctcp_acks(Exp *x, Conn *c, uint32_t k, uint32_t m)
{
    (void)x;
    c->acked += k;
    c->wa += k;
    c->wm += m;
    if (k > m) {
        uint64_t w = (uint64_t)c->cwnd + (uint64_t)(k - m) * 65536u / c->cwnd;
        c->cwnd = w > CWND_MAX ? CWND_MAX : (uint32_t)w;
    }
    if (c->acked >= c->wend) {
        uint32_t F = (uint32_t)((uint64_t)c->wm * 1024u / c->wa);
        c->alpha = c->alpha - (c->alpha >> 4) + (F >> 4);
        if (c->wm) {
            uint32_t cut = (uint32_t)(((uint64_t)c->cwnd * c->alpha) >> 11);
            c->cwnd = c->cwnd - cut < 256u ? 256u : c->cwnd - cut;
        }
        c->wend = c->sent;
        c->wa = c->wm = 0;
    }
}

/* W9c HPCC: the utilisation estimate from one ACK's telemetry against the
 * previous ACK's (the largest over the hops), folded into U. */
static void hpcc_measure(Conn *c, const uint32_t *ts, const uint32_t *tx, const uint32_t *q, const uint32_t *b)
{
    const uint64_t T = c->hT;
    uint64_t u = 0;
    uint32_t tau = 0;
    for (uint32_t i = 0; i < c->nsw; i++) {
        const uint32_t dts = ts[i] - c->L_ts[i];
        if (dts == 0) continue;                /* no time between the samples */
        const uint64_t mq = q[i] < c->L_q[i] ? q[i] : c->L_q[i];
        const uint64_t up = (65536ull * (mq * dts + (uint64_t)(tx[i] - c->L_tx[i]) * T)) / ((uint64_t)b[i] * T * dts);
        if (up > u) { u = up; tau = dts; }
    }
    if (tau > T) tau = (uint32_t)T;
    c->hU = (uint32_t)(((T - tau) * c->hU + tau * u) / T);
}

/* W9c HPCC: the new window from U; the reference window and stage move when
 * `update` (once per round trip). */
static void hpcc_window(Conn *c, int update)
{
    const uint64_t cap = (uint64_t)c->hT << 8;
    const int mult = c->hU >= HP_ETA || c->hstage >= HP_MAX_STAGE;
    uint64_t w;
    if (mult) w = (c->hU ? (uint64_t)c->hwc * HP_ETA / c->hU : cap) + c->hwai;
    else w = (uint64_t)c->hwc + c->hwai;
    if (w > cap) w = cap;
    if (w < 256) w = 256;
    c->hw = (uint32_t)w;
    if (update) {
        c->hstage = mult ? 0 : c->hstage + 1;
        c->hwc = c->hw;
    }
}

/* W9c HPCC: one ACK, carrying the telemetry of the packet it acknowledges,
 * reaches connection c's source (after acked was counted up for it). */
static void hpcc_ack(Conn *c, const uint32_t *in)
{
    const uint32_t *ts = in, *tx = in + HP_HOPS, *q = in + 2 * HP_HOPS, *b = in + 3 * HP_HOPS;
    if (c->hhave) {
        const int update = c->acked > c->hlast;
        hpcc_measure(c, ts, tx, q, b);
        hpcc_window(c, update);
        if (update) c->hlast = c->sent;
    } else {
        c->hhave = 1;
        c->hlast = c->sent;
    }
    memcpy(c->L_ts, ts, sizeof c->L_ts);
    memcpy(c->L_tx, tx, sizeof c->L_tx);
    memcpy(c->L_q, q, sizeof c->L_q);
}

/* W9b: a rate-increase event (timer or byte counter). */
static void qcn_increase(Conn *c)
{
    const uint32_t hi = c->tcnt > c->bcnt ? c->tcnt : c->bcnt;
    const uint32_t lo = c->tcnt < c->bcnt ? c->tcnt : c->bcnt;
    if (hi >= QCN_F) {
        const uint32_t add = lo > QCN_F ? (lo - QCN_F) * QCN_HAI : QCN_AI;
        c->rt = c->rt + add > QCN_ONE ? QCN_ONE : c->rt + add;
    }
    c->rc = (c->rt + c->rc) / 2;
}

/* W9b: the timer events due by tick t, in time order. */
static void qcn_timers(Conn *c, uint32_t t)
{
    for (;;) {
        const uint32_t e = c->next_inc < c->next_alpha ? c->next_inc : c->next_alpha;
        if (e > t) return;
        if (c->next_alpha == e) { c->alpha -= c->alpha >> 8; c->next_alpha += QCN_T_ALPHA; }
        if (c->next_inc == e) { c->tcnt++; qcn_increase(c); c->next_inc += QCN_T_INC; }
    }
}

/* W9b: a CNP reaches connection c's source at tick t. */
static void qcn_cnp(Conn *c, uint32_t t)
{
    qcn_timers(c, t);
    c->rt = c->rc;
    const uint32_t cut = (uint32_t)(((uint64_t)c->rc * c->alpha) >> 11);
    c->rc = c->rc - cut < QCN_RMIN ? QCN_RMIN : c->rc - cut;
    c->alpha = c->alpha - (c->alpha >> 8) + 4u;
    c->tcnt = c->bcnt = c->bsent = 0;
    c->next_inc = t + QCN_T_INC;
    c->next_alpha = t + QCN_T_ALPHA;
}

/* W9b: the source sends a packet of connection c at tick t: timers, byte
 * counter, then the pacer's next send time.  Returns the first tick at which
 * the connection may send again. */
static uint32_t qcn_sent(Conn *c, uint32_t t)
{
    qcn_timers(c, t);
    if (++c->bsent == QCN_BYTES) { c->bsent = 0; c->bcnt++; qcn_increase(c); }
    /* the pacer lags at most one tick behind its schedule, so fractional gaps
     * average out, and an idle connection gains less than one packet of
     * credit */
    const uint64_t now = ((uint64_t)t << 16) > 65535u ? ((uint64_t)t << 16) - 65535u : 0;
    c->next_fp = (c->next_fp > now ? c->next_fp : now) + (1ull << 32) / c->rc;
    return (uint32_t)((c->next_fp + 65535u) >> 16);
}

static int simulate(Exp *x, uint32_t max_ticks, orc_result *res, const orc_opts *opt)
{
    uint64_t hops = 0, delivered = 0, digest = 0;
    uint32_t flows_left = x->n_flow, t_done = 0;
    uint32_t tasks_left = x->n_task;   /* not yet finished (a compute task counts until its finish tick) */
    uint32_t max_arrive = 0, max_occ = 0;
    int rc;
    if (flows_left == 0 && tasks_left == 0) {
        res->status = ORC_OK; res->t_end = 0;
        return ORC_OK;
    }
    if (x->lb == LB_SPRAY) {
        for (uint32_t ci = 0; ci < x->n_conn; ci++) {
            Conn *c = &x->conn[ci];
            c->pkts = 0;
            for (uint32_t j = 0; j < c->nflow; j++) c->pkts += x->flow[x->conn_flows[c->flow_off + j]].size;
            c->got = (uint8_t *)calloc(c->pkts ? c->pkts : 1, 1);
            if (!c->got) return ORC_E_NOMEM;
        }
    }
    if (x->cc) {
        for (uint32_t ci = 0; ci < x->n_conn; ci++) {
            Conn *c = &x->conn[ci];
            c->cwnd = x->cwnd0 << 8;
            c->alpha = 1024;
            c->rc = c->rt = QCN_ONE;
            c->next_inc = QCN_T_INC;
            c->next_alpha = QCN_T_ALPHA;
            c->last_cnp = NONE;
            c->aq_cap = c->lat * x->R + 1;
            c->ackq = (uint32_t *)malloc(sizeof(uint32_t) * c->aq_cap);
            if (!c->ackq) return ORC_E_NOMEM;
            if (x->cc == CC_HPCC) {
                c->ackint = (uint32_t *)malloc(sizeof(uint32_t) * 4 * HP_HOPS * c->aq_cap);
                if (!c->ackint) return ORC_E_NOMEM;
                c->hT = 2 * c->lat;
                c->hw = c->hwc = c->hT << 8;
                c->hwai = (uint32_t)(((uint64_t)c->hT * 256u * (65536u - HP_ETA)) / (65536ull * HP_N));
                if (c->hwai == 0) c->hwai = 1;
                c->nsw = c->path_len - 2;
                if (c->nsw > HP_HOPS) return ORC_E_INVALID;
            }
        }
    }
    for (uint32_t t = 0; t < max_ticks; t++) {
        int busy = 0;
        /* A: ECN marks at switch arrivals, then ACKs reaching their sources */
        if (x->cc) {
            if (x->cc != CC_HPCC) ecn_mark(x, t);
            for (uint32_t ci = 0; ci < x->n_conn; ci++) {
                Conn *c = &x->conn[ci];
                uint32_t k = 0, m = 0;
                while (c->aq_n && (c->ackq[c->aq_head] >> 1) == t) {
                    m += c->ackq[c->aq_head] & 1u;
                    k++;
                    if (x->cc == CC_HPCC) {
                        c->acked++;
                        hpcc_ack(c, c->ackint + 4 * HP_HOPS * c->aq_head);
                    }
                    c->aq_head = (c->aq_head + 1) % c->aq_cap;
                    c->aq_n--;
                }
                if (c->aq_n && (c->ackq[c->aq_head] >> 1) < t) return ORC_E_INVARIANT;
                if (k && x->cc == CC_DCTCP) dctcp_acks(x, c, k, m);
                if (k && x->cc == CC_DCQCN) {
                    if (k > 1) return ORC_E_INVARIANT;     /* CNPs are 608 ticks apart */
                    qcn_cnp(c, t);
                }
            }
        }
        /* A: deliveries at hosts */
        for (uint32_t p = 0; p < x->n_ports; p++) {
            Port *pp = &x->port[p];
            if (x->layer[pp->node] != 0) continue;
            Pkt *head;
            while ((head = fifo_front(&pp->wire)) && head->arrive == t) {
                Pkt k = fifo_pop(&pp->wire);
                Conn *c = &x->conn[x->flow[k.flow].conn];
                if (opt->check) {
                    if (c->dst != pp->node) return ORC_E_INVARIANT;
                    /* ECMP keeps a connection in order: the packet belongs to its
                     * earliest flow not yet fully received */
                    if (x->lb == LB_ECMP && x->conn_flows[c->flow_off + c->recv_pos] != k.flow) return ORC_E_INVARIANT;
                }
                delivered++;
                const int notify = x->cc == CC_DCTCP || x->cc == CC_HPCC ||
                    (x->cc == CC_DCQCN && k.mark && (c->last_cnp == NONE || t - c->last_cnp >= QCN_CNP_GAP));
                if (notify) {
                    /* DCTCP: this packet's ACK; DCQCN: a CNP.  It reaches the
                     * source L ticks later */
                    if (x->cc == CC_DCQCN) c->last_cnp = t;
                    if (c->aq_n == c->aq_cap) return ORC_E_INVARIANT;
                    const uint32_t slot = (c->aq_head + c->aq_n) % c->aq_cap;
                    c->ackq[slot] = ((t + c->lat) << 1) | k.mark;
                    if (x->cc == CC_HPCC) {
                        uint32_t *d = c->ackint + 4 * HP_HOPS * slot;
                        memcpy(d, k.int_ts, sizeof k.int_ts);
                        memcpy(d + HP_HOPS, k.int_tx, sizeof k.int_tx);
                        memcpy(d + 2 * HP_HOPS, k.int_q, sizeof k.int_q);
                        memcpy(d + 3 * HP_HOPS, k.int_b, sizeof k.int_b);
                    }
                    c->aq_n++;
                    if (t + c->lat > max_arrive) max_arrive = t + c->lat;
                }
                /* packets handed to their flows now, in connection order: with
                 * spraying, this one and any later ones it was holding back */
                uint32_t n_in_order = 1;
                if (x->lb == LB_SPRAY) {
                    if (k.seq >= c->pkts || c->got[k.seq]) return ORC_E_INVARIANT;
                    c->got[k.seq] = 1;
                    n_in_order = 0;
                    while (c->rnext < c->pkts && c->got[c->rnext]) { c->rnext++; n_in_order++; }
                }
                for (uint32_t j = 0; j < n_in_order; j++) {
                    const uint32_t f = x->conn_flows[c->flow_off + c->recv_pos];
                    Flow *fl = &x->flow[f];
                    if (++fl->recvd < fl->size) continue;
                    fl->rd = t;
                    c->recv_pos++;
                    digest += mix64(((uint64_t)f << 32) | t);
                    if (t > t_done) t_done = t;
                    flows_left--;
                    uint32_t tk = x->flow_task[f];
                    if (tk != NONE && --x->task[tk].left == 0) {
                        x->task[tk].finish = t;     /* the collective's last flow arrived */
                        tasks_left--;
                    }
                }
            }
            if (pp->wire.count && fifo_front(&pp->wire)->arrive < t) return ORC_E_INVARIANT;
        }
        /* Schedule: a task starts at the first tick by which all its
         * predecessors have finished; a compute or intra-server task finishes
         * its duration later (at least one tick, so no task both starts and
         * finishes within one tick) */
        for (uint32_t k = 0; k < x->n_task; k++) {
            Task *tk = &x->task[k];
            if (tk->start != NONE) {
                if (tk->type != TASK_COLL && tk->finish == t) tasks_left--;
                continue;
            }
            int ok = 1;
            for (uint32_t q = 0; q < tk->npred && ok; q++) {
                uint32_t fin = x->task[x->task_pred[tk->pred_off + q]].finish;
                if (fin == NONE || fin > t) ok = 0;
            }
            if (!ok) continue;
            tk->start = t;
            busy = 1;
            if (tk->type != TASK_COLL) {
                tk->finish = t + tk->dur;
                if (tk->finish > max_arrive) max_arrive = tk->finish;
                if (tk->finish > t_done) t_done = tk->finish;
            }
        }
        /* B: activation.  Only the first not yet active flow of a connection can
         * have all its predecessors met: every later one waits (SEND) on it. */
        for (uint32_t ci = 0; ci < x->n_conn; ci++) {
            Conn *c = &x->conn[ci];
            if (c->cur >= c->nflow) continue;
            Flow *fl = &x->flow[x->conn_flows[c->flow_off + c->cur]];
            if (fl->active) continue;
            int ok = 1;
            for (uint32_t k = 0; k < fl->npred; k++) {
                uint32_t when;
                if (fl->pkind[k] == PRED_TASK) when = x->task[fl->pred[k]].start;
                else when = fl->pkind[k] == PRED_RECV ? x->flow[fl->pred[k]].rd : x->flow[fl->pred[k]].sd;
                if (when == NONE || when > t) { ok = 0; break; }
            }
            if (ok) { fl->active = 1; fl->act = t; busy = 1; }
        }
        /* C: credit snapshot */
        for (uint32_t p = 0; p < x->n_ports; p++) {
            Port *pp = &x->port[p];
            if (x->layer[pp->peer_node] == 0) pp->credit = INT64_MAX;
            else pp->credit = (int64_t)x->Q - (int64_t)x->port[pp->peer_port].occ;
        }
        /* W9c: every switch egress's backlog at the start of the tick, for telemetry */
        if (x->cc == CC_HPCC)
            for (uint32_t n = 0; n < x->n_nodes; n++) {
                if (x->layer[n] == 0) continue;
                for (uint32_t o = 0; o < x->port_off[n + 1] - x->port_off[n]; o++)
                    x->port[x->port_off[n] + o].bl = egress_backlog(x, n, o, t);
            }
        /* D: rounds of grants; decide on the state at the start of the round, then apply */
        for (uint32_t m = 0; m < x->R; m++) {
            for (uint32_t p = 0; p < x->n_ports; p++) {
                Port *pp = &x->port[p];
                pp->granted = NONE;
                if (!pp->alive || m >= pp->rate || pp->credit <= 0) continue;
                uint32_t node = pp->node;
                uint32_t me = p - x->port_off[node];
                if (x->layer[node] == 0) {
                    uint32_t n_in = x->host_conn_off[node + 1] - x->host_conn_off[node];
                    for (uint32_t j = 0; j < n_in; j++) {
                        uint32_t idx = (pp->rr + j) % n_in;
                        Conn *c = &x->conn[x->host_conn[x->host_conn_off[node] + idx]];
                        if (c->cur >= c->nflow) continue;
                        Flow *fl = &x->flow[x->conn_flows[c->flow_off + c->cur]];
                        if (x->cc == CC_DCTCP && c->sent - c->acked >= (c->cwnd >> 8)) continue;   /* window full */
                        if (x->cc == CC_HPCC && c->sent - c->acked >= (c->hw >> 8)) continue;      /* window full */
                        if (x->cc == CC_DCQCN && ((uint64_t)t << 16) < c->next_fp) continue;        /* paced */
                        if (fl->active && fl->sent < fl->size) { pp->granted = idx; break; }
                    }
                } else {
                    uint32_t deg = x->port_off[node + 1] - x->port_off[node];
                    for (uint32_t j = 0; j < deg; j++) {
                        uint32_t i = (pp->rr + j) % deg;
                        Pkt *head = fifo_front(&x->port[x->port_off[node] + i].voq[me]);
                        if (head && head->arrive <= t) { pp->granted = i; break; }
                    }
                }
            }
            for (uint32_t p = 0; p < x->n_ports; p++) {
                Port *pp = &x->port[p];
                if (pp->granted == NONE) continue;
                uint32_t node = pp->node;
                busy = 1;
                if (x->layer[node] == 0) {
                    uint32_t n_in = x->host_conn_off[node + 1] - x->host_conn_off[node];
                    uint32_t ci = x->host_conn[x->host_conn_off[node] + pp->granted];
                    Conn *c = &x->conn[ci];
                    uint32_t f = x->conn_flows[c->flow_off + c->cur];
                    Flow *fl = &x->flow[f];
                    if (out_port(x, c, 0) != p) return ORC_E_INVARIANT;
                    rc = transmit(x, p, NULL, f, 0, 0, c->sent, t, &hops, &max_arrive, &max_occ);
                    if (rc) return rc;
                    fl->sent++;
                    c->sent++;
                    if (x->cc == CC_DCQCN) {
                        const uint32_t next_tick = qcn_sent(c, t);
                        if (next_tick > max_arrive) max_arrive = next_tick;
                    }
                    if (fl->sent == fl->size) { fl->sd = t + 1; c->cur++; }
                    pp->rr = (pp->granted + 1) % n_in;
                } else {
                    uint32_t deg = x->port_off[node + 1] - x->port_off[node];
                    uint32_t me = p - x->port_off[node];
                    Port *in = &x->port[x->port_off[node] + pp->granted];
                    Pkt k = fifo_pop(&in->voq[me]);
                    in->occ--;
                    const Conn *c = &x->conn[x->flow[k.flow].conn];
                    if (opt->check && x->lb == LB_ECMP && out_port(x, c, k.hop) != p) return ORC_E_INVARIANT;
                    rc = transmit(x, p, &k, k.flow, k.hop, k.mark, k.seq, t, &hops, &max_arrive, &max_occ);
                    if (rc) return rc;
                    pp->rr = (pp->granted + 1) % deg;
                }
                pp->credit--;
            }
        }
        /* E: completion / static state */
        if (flows_left == 0 && tasks_left == 0) {
            res->status = ORC_OK;
            res->t_end = t_done;
            res->pkt_hops = hops; res->delivered = delivered; res->digest = digest;
            res->max_occupancy = max_occ;
            return ORC_OK;
        }
        if (!busy && max_arrive <= t) {
            res->status = ORC_S_DEADLOCK;
            res->t_end = t;
            res->pkt_hops = hops; res->delivered = delivered; res->digest = digest;
            res->max_occupancy = max_occ;
            return ORC_OK;
        }
    }
    res->status = ORC_S_INCOMPLETE;
    res->t_end = max_ticks;
    res->pkt_hops = hops; res->delivered = delivered; res->digest = digest;
    res->max_occupancy = max_occ;
    return ORC_OK;
}

/* ------------------------------------------------------------- interface */

/* Number of flows and connections of experiment e (validates the workload). */
int orc_count(const orc_batch *b, uint32_t e, uint64_t *n_flows, uint64_t *n_conns)
{
    if (e >= b->n_exp) return ORC_E_INVALID;
    return count_workload(b, e, n_conns, n_flows);
}

/* Runs experiment e for at most max_ticks ticks.  Optional per-flow outputs
 * (NONE where the event did not happen): RD, activation tick, SD; per task:
 * start and finish ticks.  Returns a
 * negative error code, or ORC_OK with the status in res->status. */
int orc_run(const orc_batch *b, uint32_t e, uint32_t max_ticks, uint32_t check, orc_result *res,
            uint32_t *flow_rd, uint32_t *flow_act, uint32_t *flow_sd, uint32_t *task_start, uint32_t *task_finish)
{
    Exp x;
    memset(&x, 0, sizeof(x));
    memset(res, 0, sizeof(*res));
    if (e >= b->n_exp) return ORC_E_INVALID;
    x.Q = b->exp_queue_pkts[e];
    x.seed = b->exp_ecmp_seed[e];
    if (x.Q < 1) return ORC_E_INVALID;
    x.cc = b->exp_cc ? b->exp_cc[e] : CC_NONE;
    if (x.cc > CC_HPCC) return ORC_E_INVALID;
    x.lb = b->exp_lb ? b->exp_lb[e] : LB_ECMP;
    /* sprayed packets of one connection see different path latencies, which
     * the ACK timing of W9 does not describe */
    if (x.lb > LB_SPRAY || (x.lb == LB_SPRAY && x.cc != CC_NONE)) return ORC_E_INVALID;
    if (x.cc) {
        x.ecn_k = b->exp_ecn_k[e];
        x.cwnd0 = b->exp_cwnd0[e];
        if (x.cc == CC_DCTCP && (x.cwnd0 < 1 || x.cwnd0 > 65535)) return ORC_E_INVALID;
    }
    int rc = build_topology(b, e, &x);
    if (!rc) rc = build_workload(b, e, &x);
    if (!rc) rc = build_routes(&x);
    orc_opts opt;
    opt.flow_rd = flow_rd; opt.flow_act = flow_act; opt.flow_sd = flow_sd; opt.check = check;
    if (!rc) {
        res->n_flows = x.n_flow;
        res->n_conns = x.n_conn;
        rc = simulate(&x, max_ticks, res, &opt);
    }
    if (!rc) {
        for (uint32_t f = 0; f < x.n_flow; f++) {
            if (flow_rd) flow_rd[f] = x.flow[f].rd;
            if (flow_act) flow_act[f] = x.flow[f].act;
            if (flow_sd) flow_sd[f] = x.flow[f].sd;
        }
        for (uint32_t k = 0; k < x.n_task; k++) {
            if (task_start) task_start[k] = x.task[k].start;
            if (task_finish) task_finish[k] = x.task[k].finish;
        }
    }
    exp_free(&x);
    return rc;
}

/* Per-connection description for tests: source, destination, number of links
 * on its path, and the global port index used at each path position (up to
 * max_len entries per connection; NONE after the end). */
int orc_paths(const orc_batch *b, uint32_t e, uint32_t *conn_src, uint32_t *conn_dst,
              uint32_t *conn_links, uint32_t *path_ports, uint32_t max_len)
{
    Exp x;
    memset(&x, 0, sizeof(x));
    if (e >= b->n_exp) return ORC_E_INVALID;
    x.Q = b->exp_queue_pkts[e];
    x.seed = b->exp_ecmp_seed[e];
    int rc = build_topology(b, e, &x);
    if (!rc) rc = build_workload(b, e, &x);
    if (!rc) rc = build_routes(&x);
    if (!rc) {
        for (uint32_t c = 0; c < x.n_conn; c++) {
            Conn *cn = &x.conn[c];
            conn_src[c] = cn->src; conn_dst[c] = cn->dst; conn_links[c] = cn->path_len - 1;
            for (uint32_t h = 0; h < max_len; h++)
                path_ports[(size_t)c * max_len + h] =
                    h + 1 < cn->path_len ? out_port(&x, cn, h) : NONE;
        }
    }
    exp_free(&x);
    return rc;
}

/* Per-flow description for tests: connection and size of every flow. */
int orc_flows(const orc_batch *b, uint32_t e, uint32_t *flow_conn, uint32_t *flow_size)
{
    Exp x;
    memset(&x, 0, sizeof(x));
    if (e >= b->n_exp) return ORC_E_INVALID;
    x.Q = b->exp_queue_pkts[e] ? b->exp_queue_pkts[e] : 1;
    int rc = build_topology(b, e, &x);
    if (!rc) rc = build_workload(b, e, &x);
    if (!rc)
        for (uint32_t f = 0; f < x.n_flow; f++) { flow_conn[f] = x.flow[f].conn; flow_size[f] = x.flow[f].size; }
    exp_free(&x);
    return rc;
}

uint32_t orc_fmix32(uint32_t h) { return fmix32(h); }

/* W9c's per-connection window machine on its own, for pins: a fresh
 * connection with base round trip T and nsw switches on its path receives n
 * ACKs in order; ACK i comes when the source has sent sent[i] packets and
 * carries telemetry tel[4 nsw i ..] (ticks, packets sent, backlogs, rates,
 * nsw each).  After each, state[4 i ..] = U, W, Wc and the stage. */
int orc_hpcc_script(uint32_t T, uint32_t nsw, uint32_t n, const uint32_t *sent, const uint32_t *tel, uint32_t *state)
{
    if (T == 0 || nsw == 0 || nsw > HP_HOPS) return ORC_E_INVALID;
    Conn c;
    memset(&c, 0, sizeof c);
    c.hT = T;
    c.hw = c.hwc = T << 8;
    c.hwai = (uint32_t)(((uint64_t)T * 256u * (65536u - HP_ETA)) / (65536ull * HP_N));
    if (c.hwai == 0) c.hwai = 1;
    c.nsw = nsw;
    for (uint32_t i = 0; i < n; i++) {
        uint32_t in[4 * HP_HOPS] = {0};
        for (uint32_t k = 0; k < 4; k++)
            for (uint32_t h = 0; h < nsw; h++) in[k * HP_HOPS + h] = tel[4 * nsw * i + k * nsw + h];
        for (uint32_t h = 0; h < nsw; h++) if (in[3 * HP_HOPS + h] == 0) return ORC_E_INVALID;
        if (sent[i] < c.acked + 1) return ORC_E_INVALID;
        c.sent = sent[i];
        c.acked++;
        hpcc_ack(&c, in);
        state[4 * i] = c.hU;
        state[4 * i + 1] = c.hw;
        state[4 * i + 2] = c.hwc;
        state[4 * i + 3] = c.hstage;
    }
    return ORC_OK;
}

/* W9b's per-connection rate machine on its own, for pins: a fresh
 * connection receives n events in tick order, what[i] = 0 a CNP and 1 a
 * packet sent, at tick[i]; after each, state[4 i ..] = RC, RT, alpha and the
 * first tick the pacer allows the next packet (the tick itself after a CNP). */
int orc_qcn_script(uint32_t n, const uint32_t *tick, const uint8_t *what, uint32_t *state)
{
    Conn c;
    memset(&c, 0, sizeof c);
    c.rc = c.rt = QCN_ONE;
    c.alpha = 1024;
    c.next_inc = QCN_T_INC;
    c.next_alpha = QCN_T_ALPHA;
    for (uint32_t i = 0; i < n; i++) {
        if (i && tick[i] < tick[i - 1]) return ORC_E_INVALID;
        uint32_t next = tick[i];
        if (what[i] == 0) qcn_cnp(&c, tick[i]);
        else if (what[i] == 1) next = qcn_sent(&c, tick[i]);
        else return ORC_E_INVALID;
        state[4 * i] = c.rc;
        state[4 * i + 1] = c.rt;
        state[4 * i + 2] = c.alpha;
        state[4 * i + 3] = next;
    }
    return ORC_OK;
}
uint64_t orc_mix64(uint64_t z) { return mix64(z); }
