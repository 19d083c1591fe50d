/*
 * msim.h -- C ABI of the batched packet-level network simulator for AMD MI355X
 * (gfx950).
 *
 * One process simulates a whole batch of independent experiments on one GPU:
 * the single-process multi-experiment strategy of Multiverse ("Accelerating
 * Design Space Exploration for LLM Training Systems with Multi-experiment
 * Parallel Simulation", section 2.2).  Each experiment is a switched topology,
 * a collective-communication workload and a few parameters, as the user lists
 * them in Multiverse's usage model (section 3.1 "Architecture").  The network
 * part of that system -- point-to-point flows produced from NCCL's collective
 * algorithms, a lockstep packet-level simulation with pull-based forwarding
 * (section 4.2) and one kernel launch per batch (section 4.3) -- is what this
 * library computes.  Collective shapes: ring all-reduce and ring all-gather cut
 * into NC channels and chunks of size C (AutoCCL, "Automated Collective
 * Communication Tuning", section 2.3), the K-partition pipelined broadcast
 * (AlpaComm, "On Optimizing the Communication of Model Parallelism", section
 * 3.1, Fig. 3d), and explicit flows for sparse all-to-all traffic.
 *
 * Conventions
 *  - Plain C, fixed-width integers, no exceptions cross this boundary.
 *  - Every entry point returns MSIM_OK (0), a positive run status, or a negative
 *    error code; msim_last_error() gives a message for the last failure.
 *  - Host arrays passed in are owned by the caller and only read during the
 *    call.  Device memory (the workspace) is allocated by the caller and must
 *    outlive the context; the library allocates no device memory itself.
 *  - A context is used from one host thread at a time.
 *  - Sizing follows compiling: msim_create compiles on the host, then
 *    msim_workspace_size and msim_bind size and fill the caller's workspace.
 *  - msim_run only enqueues; the run status (MSIM_S_*) comes from msim_results.
 *  - Results go to host arrays.  Per-flow ticks are kept only for the
 *    experiments named at create (msim_options.record_exp).
 *  - An experiment's tick stops at 0xFFFFFFF0; one that reaches it stays
 *    MSIM_EXP_INCOMPLETE (there is no overflow error).
 *
 * Time is counted in integer ticks (one tick = the smallest link delay,
 * Multiverse section 5); data in whole packets of exp_pkt_bytes bytes.
 */
#ifndef MSIM_H
#define MSIM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSIM_ABI_VERSION 5u

/* return codes */
#define MSIM_OK 0
#define MSIM_S_INCOMPLETE 1      /* msim_run: some experiment hit its tick budget */
#define MSIM_S_DEADLOCK 2        /* msim_run: some experiment reached a static, unfinished state */
#define MSIM_E_INVALID_SPEC (-1) /* the batch violates a rule listed below */
#define MSIM_E_UNROUTABLE (-2)   /* a connection has no up/down path over alive cables */
#define MSIM_E_WORKSPACE (-3)    /* workspace missing, too small or misaligned */
#define MSIM_E_HIP (-4)          /* a HIP runtime call failed */
#define MSIM_E_ARG (-5)          /* bad argument (null pointer, index out of range) */
#define MSIM_E_STATE (-6)        /* call out of order (e.g. run before bind) */
#define MSIM_E_LIMIT (-7)        /* an input exceeds a compiled-in limit */

/* per-experiment status (msim_results) */
#define MSIM_EXP_DONE 0          /* every flow received; tick = completion tick */
#define MSIM_EXP_INCOMPLETE 1    /* tick budget spent; tick = ticks simulated so far */
#define MSIM_EXP_DEADLOCK 2      /* tick = first tick of the static state */
#define MSIM_EXP_FAULT 3         /* internal invariant broken (a library bug); results void */

/* collective kinds (coll_type) */
#define MSIM_COLL_RING_ALLREDUCE 1
#define MSIM_COLL_RING_ALLGATHER 2
#define MSIM_COLL_PIPE_BROADCAST 3
#define MSIM_COLL_RING_REDUCESCATTER 4   /* Multiverse section 5 lists it among its collectives */
#define MSIM_COLL_TREE_ALLREDUCE 5       /* AutoCCL section 4.1: tree (log2 N) against ring (2(N-1)) */
#define MSIM_COLL_SENDRECV 6             /* AlpaComm section 3.1, Figure 3a: one source, receivers in turn */
#define MSIM_NO_GATE 0xFFFFFFFFu

/* task kinds (task_type): the System Simulator's task graph, Multiverse
 * sections 3.1 and 3.2 (Schedule, AnalyticalSys) */
#define MSIM_TASK_COMPUTE 0      /* lasts task_ticks ticks */
#define MSIM_TASK_INTRA 1        /* intra-server collective: task_ticks + ceil(task_bytes / task_beta)
                                    ticks, the alpha + size / beta model of section 4.1 */
#define MSIM_TASK_COLL 2         /* the workload's collective task_coll, simulated packet by packet */

/* congestion control (exp_cc): Multiverse section 3.2 gives flows
 * congestion-control variables and closes each simulation step with an ACK
 * system; section 5 names DCTCP among the algorithms it integrates */
#define MSIM_CC_NONE 0
#define MSIM_CC_DCTCP 1          /* ECN marks at switches, ACKs, a DCTCP window per connection */
#define MSIM_CC_DCQCN 2          /* ECN marks at switches, CNPs, a DCQCN rate per connection */
#define MSIM_CC_HPCC 3           /* in-band telemetry at switches, ACKs, an HPCC window per connection */
#define MSIM_MAX_CWND 65535      /* packets */

/* load balancing (exp_lb), Multiverse section 5: ECMP and packet spraying */
#define MSIM_LB_ECMP 0           /* one route per connection (hash of the connection) */
#define MSIM_LB_SPRAY 1          /* every packet chooses at every switch (hash of connection and sequence) */

/* compiled-in limits */
#define MSIM_MAX_RATE 4          /* packets per tick per link direction */
#define MSIM_MAX_DELAY 15        /* ticks per cable */
#define MSIM_MAX_SWITCH_PORTS 16
#define MSIM_MAX_SWITCH_HOPS 8   /* switches on one path */
#define MSIM_MAX_QUEUE 255       /* packets per switch ingress buffer */

/*
 * A batch of experiments.  Topologies and workloads are listed once and shared
 * by reference; CSR offset arrays have one entry more than the items they
 * index.  All arrays are host memory.
 *
 * Topology t: nodes topo_node_off[t] .. topo_node_off[t+1]-1 with node_layer
 *   0 = host, 1..3 = switch layers; cables topo_cable_off[t] ..
 *   topo_cable_off[t+1]-1 joining nodes cable_a / cable_b (indices local to the
 *   topology), with packets/tick cable_rate_ab (a to b) and cable_rate_ba,
 *   delay in ticks (both directions) and an alive flag (0 = failed cable).  A
 *   node's ports are numbered in the order its cables are listed.  Rules: every
 *   host has exactly one cable; a cable joins nodes of different layers; rates
 *   1..MSIM_MAX_RATE; delays 1..MSIM_MAX_DELAY; a switch has at most
 *   MSIM_MAX_SWITCH_PORTS ports.
 * Workload w: collectives work_coll_off[w] .. work_coll_off[w+1]-1, each with
 *   coll_type, coll_bytes (all-gather: total output size; reduce-scatter:
 *   total input size; send/recv: bytes each receiver gets), coll_nc channels
 *   (rings, trees), coll_chunk_bytes (rings, trees; a whole number of
 *   packets), coll_k partitions (broadcast; 1 <= K <= packets), coll_gate
 *   (MSIM_NO_GATE, or for a ring the index within the workload of an earlier
 *   send/recv whose receivers are exactly the ring's members in ring order:
 *   each rank then starts once its piece of that send/recv has arrived) and
 *   members coll_member_off[c] .. coll_member_off[c+1]-1 in member_host (ring
 *   order; broadcast chain or send/recv with the source first; tree in heap
 *   order, member 0 the root, the parent of member i being member (i-1)/2;
 *   distinct hosts, at least 2); then explicit flows
 *   work_xflow_off[w] .. work_xflow_off[w+1]-1 (source host, destination host,
 *   packets >= 1).  Every ring channel must carry at least as many packets as
 *   the ring has members, every tree channel at least one packet.
 *   Tasks (optional; work_task_off NULL = none): tasks work_task_off[w] ..
 *   work_task_off[w+1]-1 of workload w, in topological order, with task_type,
 *   task_ticks, task_bytes, task_beta, task_coll (a collective index within
 *   the workload; each collective named by at most one task) and predecessors
 *   task_pred[task_pred_off[k] .. task_pred_off[k+1]-1] (task indices within
 *   the workload, each below k).  A task starts at the first tick by which
 *   every predecessor has finished; a compute or intra-server task finishes its
 *   duration (>= 1 tick) later, a collective task when its last flow arrives.
 *   A collective a task names starts with that task; the others start at tick
 *   0.  An experiment with tasks runs on the general path.
 * Experiment e: topology exp_topo[e], workload exp_work[e], switch ingress
 *   buffer exp_queue_pkts[e] packets (1..MSIM_MAX_QUEUE), ECMP seed
 *   exp_ecmp_seed[e], packet size exp_pkt_bytes[e] bytes, congestion control
 *   exp_cc[e] (exp_cc NULL = MSIM_CC_NONE for all).  With MSIM_CC_DCTCP
 *   (DCTCP, Alizadeh et al., SIGCOMM 2010, in integer arithmetic):
 *   - a packet reaching a switch at tick t is ECN-marked when at least
 *     exp_ecn_k[e] packets for the same egress had arrived there before t and
 *     not left before t; the mark stays with the packet;
 *   - a packet delivered at t acknowledges itself at its connection's source at
 *     t + L, L the sum of the path's link delays; ACKs use no link capacity;
 *   - each connection keeps a window cwnd (1/256 packet; initially
 *     exp_cwnd0[e] packets, 1..MSIM_MAX_CWND) and alpha (1/1024; initially 1),
 *     and sends only while packets sent - packets acknowledged < floor(cwnd);
 *   - the k ACKs (m marked) of a tick add (k - m) * 65536 / cwnd to cwnd (at
 *     most MSIM_MAX_CWND packets); when the acknowledged count reaches the
 *     window end, alpha = alpha - alpha/16 + F/16 (F = 1024 * marked /
 *     acknowledged in the window), cwnd = max(1 packet, cwnd - cwnd * alpha /
 *     2048) if any was marked, and the next window ends at the packets sent so
 *     far (the first window ends at 0).
 *   With MSIM_CC_DCQCN (DCQCN, Zhu et al., SIGCOMM 2015, in integer
 *   arithmetic; exp_cwnd0 unused, may be NULL):
 *   - the same ECN marks (threshold exp_ecn_k[e]);
 *   - a marked packet delivered at t sends a CNP to its connection's source,
 *     arriving at t + L, unless the connection's previous CNP was sent less
 *     than 608 ticks before t;
 *   - each connection keeps a rate RC and target RT (1/65536 packet per tick,
 *     initially 65536: the line rate is one packet per tick) and alpha (1/1024,
 *     initially 1).  A CNP at t: RT = RC, RC = max(64, RC - RC * alpha / 2048),
 *     alpha = alpha - alpha/256 + 4, and the stage counters and both timers
 *     restart at t.  Every 640 ticks without a CNP alpha loses alpha/256; every
 *     640 ticks and every 2560 packets sent an increase event raises its stage
 *     count, then: both stages below 5, RT stays; both above 5, RT += 160 *
 *     (min stage - 5); else RT += 64; RT <= 65536; RC = (RT + RC) / 2.  Timer
 *     events due by t come before a CNP or send at t, alpha's before the
 *     increase on the same tick;
 *   - a connection sends only at ticks t with t * 65536 >= its next send time
 *     N (initially 0); a packet sent at t sets N = max(N, t * 65536 - 65535) +
 *     floor(2^32 / RC).
 *   With MSIM_CC_HPCC (HPCC, Li et al., SIGCOMM 2019, Algorithm 1, in integer
 *   arithmetic; exp_ecn_k and exp_cwnd0 unused, may be NULL; no ECN marks):
 *   - a packet leaving a switch egress at tick t records, for that switch,
 *     (t, packets the egress has sent including this one, the egress's
 *     backlog at the start of t as for ECN, the egress rate); each packet is
 *     ACKed as under DCTCP and the ACK carries the packet's records;
 *   - each connection keeps T = 2 L, a window W and reference window Wc (1/256
 *     packet, initially T packets, always 1 .. T packets), U (1/65536,
 *     initially 0) and an increase stage; W_AI = floor(T * 256 * 3277 /
 *     (65536 * 16)), at least 1; it sends only while sent - acked < floor(W);
 *   - ACKs are applied one by one in sequence order.  The first only records
 *     its telemetry and sets the update mark to the packets sent.  A later
 *     one: per switch i with dts = t_i - t_i(previous ACK) > 0, u_i =
 *     floor(65536 (min(q_i, q_i prev) dts + (n_i - n_i prev) T) / (rate_i T
 *     dts)); u and tau start at 0 and, switch by switch in path order, u_i >
 *     u replaces them with (u_i, dts); tau is capped at T; U = floor(((T -
 *     tau) U + tau u) / T).
 *     If U >= 62259 (0.95) or the stage is 5: W = floor(Wc * 62259 / U) +
 *     W_AI (W = T packets if U = 0), else W = Wc + W_AI, then clamped; if
 *     the acknowledged count exceeds the update mark, Wc = W, the stage goes
 *     to 0 (first case) or up by 1, and the mark becomes the packets sent;
 *   - at most 8 switches per path (MSIM_MAX_SWITCH_HOPS).
 *   An experiment with congestion control runs on the general path.
 *   Load balancing exp_lb[e] (exp_lb NULL = MSIM_LB_ECMP for all): with
 *   MSIM_LB_SPRAY a packet with sequence number s (packets its connection sent
 *   before it) leaves switch n through cand[fmix32(key ^ fmix32(n ^ seed)) mod
 *   |cand|], key = connection ^ fmix32(s + 1), cand the same equal-cost
 *   egresses as ECMP (sorted by port; only downward once the packet has moved
 *   down a layer).  Each connection still delivers in order: a flow is received
 *   once all its packets and all earlier ones of its connection have arrived.
 *   Spraying runs on the general path, and not together with congestion
 *   control (MSIM_E_INVALID_SPEC).
 */
typedef struct msim_batch_spec {
    uint32_t version;            /* MSIM_ABI_VERSION */
    uint32_t n_topo, n_work, n_exp;
    const uint32_t *topo_node_off;
    const uint8_t *node_layer;
    const uint32_t *topo_cable_off;
    const uint32_t *cable_a, *cable_b;
    const uint8_t *cable_rate_ab, *cable_rate_ba, *cable_delay, *cable_alive;
    const uint32_t *work_coll_off;
    const uint8_t *coll_type;
    const uint64_t *coll_bytes;
    const uint32_t *coll_nc, *coll_chunk_bytes, *coll_k;
    const uint32_t *coll_member_off, *member_host;
    const uint64_t *work_xflow_off;
    const uint32_t *xflow_src, *xflow_dst, *xflow_pkts;
    const uint32_t *exp_topo, *exp_work, *exp_queue_pkts, *exp_ecmp_seed, *exp_pkt_bytes;
    const uint32_t *coll_gate;   /* one per collective; NULL = no gates */
    const uint32_t *work_task_off;
    const uint8_t *task_type;
    const uint32_t *task_ticks;
    const uint64_t *task_bytes;
    const uint32_t *task_beta, *task_coll;
    const uint32_t *task_pred_off, *task_pred;
    const uint8_t *exp_cc;       /* one per experiment; NULL = no congestion control */
    const uint32_t *exp_ecn_k, *exp_cwnd0;
    const uint8_t *exp_lb;       /* one per experiment; NULL = MSIM_LB_ECMP */
} msim_batch_spec;

/* Options for msim_create.  Zero-initialise and set what you need. */
typedef struct msim_options {
    uint32_t version;            /* MSIM_ABI_VERSION */
    uint32_t n_record;           /* experiments whose per-flow ticks are kept */
    const uint32_t *record_exp;  /* their indices (host array of n_record) */
    uint32_t host_threads;       /* threads for the host-side compile; 0 = all cores */
    uint32_t force_global;       /* 1: keep experiment state in HBM even where it fits in LDS */
    uint32_t block_threads;      /* 0 = automatic; else 64..1024, multiple of 64 */
    uint32_t no_ring_path;       /* 1: run ring-only experiments on the general compact kernels too
                                    (msim_megakernel_c8h_r1 and kin) instead of msim_megakernel_ring */
    uint32_t reserved[7];
} msim_options;

typedef struct msim_ctx msim_ctx; /* opaque; owned by the library */

/*
 * Validates the batch and compiles it on the host: ports and cables, up/down
 * shortest-path ECMP routes (Multiverse section 5: ECMP load balancing), the
 * collectives' point-to-point connections and flow schedules (Multiverse
 * section 3.1: the system simulator turns NCCL's collective algorithms into
 * point-to-point flows), and the experiment-major state layout.  No device
 * memory is touched.  On error *out is NULL and the return code says why
 * (MSIM_E_INVALID_SPEC, MSIM_E_UNROUTABLE, MSIM_E_LIMIT); the message is
 * available from msim_last_error(NULL) on the same thread.
 */
int msim_create(const msim_batch_spec *spec, const msim_options *opts, msim_ctx **out);

/* Bytes of device workspace msim_bind needs (256-byte aligned start): the
 * experiment-major state store of every experiment of the batch (Multiverse
 * section 3.3: the state of all experiments kept in one centralised store, as
 * columns the simulation steps work on), its pristine copy for msim_reset, and
 * the per-flow tick records of the recorded experiments.  The caller allocates
 * it (device memory from its own allocator, e.g. a torch tensor) and keeps it
 * alive as long as the context.  MSIM_E_ARG for a NULL argument. */
int msim_workspace_size(const msim_ctx *ctx, uint64_t *bytes);

/*
 * Binds a caller-owned device buffer of at least msim_workspace_size bytes and
 * uploads the compiled batch into it on the given stream (a hipStream_t; NULL =
 * the default stream), then waits for the upload.  Binding again re-uploads.
 */
int msim_bind(msim_ctx *ctx, void *dev_workspace, uint64_t ws_bytes, void *hip_stream);

/*
 * Launches the simulation of every unfinished experiment for at most max_ticks
 * more ticks each, as one kernel launch per kernel kind present in the batch on
 * hip_stream (asynchronous; one launch per batch, Multiverse section 4.3).  In a
 * batch where some experiment moves 2^32 or more packet-hops, a max_ticks above
 * 2^30 is split into consecutive launches of at most 2^30 ticks, with the same
 * result.  Experiments are independent; their state
 * stays in the workspace between calls, so several calls continue where the
 * previous one stopped.  Returns MSIM_OK once enqueued; per-experiment outcome
 * comes from msim_results.  flags: reserved, pass 0 (per-flow recording is
 * chosen per experiment at msim_create, see msim_options.record_exp).
 */
int msim_run(msim_ctx *ctx, uint32_t max_ticks, void *hip_stream, uint32_t flags);

/*
 * msim_run_noalloc: msim_run for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, same kernels, same results as msim_run; the
 * difference is where the kernels' experiment queue counters (one per kernel
 * launch of the call) live: in a static device array of MSIM_NOALLOC_LAUNCHES
 * 32-bit words that the library holds on each GPU until the process ends,
 * instead of the workspace header.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); it zeroes the counters it uses with
 * a kernel on hip_stream.  The workspace's device must be current.  A call
 * needing more launches than MSIM_NOALLOC_LAUNCHES (one per kernel kind present
 * in the batch, times ceil(max_ticks / 2^30) when an experiment moves 2^32 or
 * more packet-hops) returns MSIM_E_LIMIT and launches nothing.  Every call on
 * one GPU shares that GPU's counters: calls that overlap on one GPU (other
 * streams, other host threads, other contexts) race and must not be made.
 */
#define MSIM_NOALLOC_LAUNCHES 64u
int msim_run_noalloc(msim_ctx *ctx, uint32_t max_ticks, void *hip_stream, uint32_t flags);

/* Restores every experiment to tick 0 (asynchronous, on hip_stream). */
int msim_reset(msim_ctx *ctx, void *hip_stream);

/*
 * The outcome of every experiment: Multiverse section 3.1 has the network
 * simulator report each flow's completion back to the system simulator; per
 * experiment that is the completion tick (the last flow's arrival), and the
 * digest condenses every flow's completion tick into one number.
 * Waits for hip_stream, then copies per-experiment results to host arrays
 * (any pointer may be NULL to skip it), each of n_exp entries:
 *   exp_status    MSIM_EXP_*;
 *   exp_tick      completion tick (DONE), first static tick (DEADLOCK) or ticks
 *                 simulated so far (INCOMPLETE);
 *   exp_pkt_hops  packet transmissions on every link, host NICs included;
 *   exp_delivered packets received by hosts;
 *   exp_digest    sum over flows f of mix64((f << 32) | RD_f) mod 2^64, mix64
 *                 being SplitMix64's output function and RD_f the tick the last
 *                 packet of flow f arrived (flows not yet received add nothing).
 * Returns MSIM_S_DEADLOCK if any experiment deadlocked, else MSIM_S_INCOMPLETE
 * if any is unfinished, else MSIM_OK.
 */
int msim_results(msim_ctx *ctx, void *hip_stream, uint8_t *exp_status, uint32_t *exp_tick,
                 uint64_t *exp_pkt_hops, uint64_t *exp_delivered, uint64_t *exp_digest);

/* Number of flows of experiment exp: the point-to-point flows the collective
 * algorithms are turned into (Multiverse section 3.1; AutoCCL section 2.3 for
 * a ring's channels and chunks).  Flows are numbered per experiment: the
 * collectives in input order -- a ring by channel, round, step, rank; a
 * broadcast by hop, partition -- then the explicit flows.  MSIM_E_ARG for an
 * experiment index out of range. */
int msim_flow_count(const msim_ctx *ctx, uint32_t exp, uint64_t *n_flows);

/*
 * Flow completion as Multiverse section 3.1 reports it, flow by flow.
 * Per-flow ticks of a recorded experiment (listed in msim_options.record_exp):
 * arrival of the last packet (rd), activation (act) and last send + 1 (sd),
 * 0xFFFFFFFF where the event has not happened.  Arrays of n_flows entries, or
 * NULL.  Waits for hip_stream first.  MSIM_E_ARG if exp was not recorded.
 */
int msim_flow_ticks(msim_ctx *ctx, uint32_t exp, void *hip_stream, uint32_t *rd, uint32_t *act,
                    uint32_t *sd);

/* Number of tasks of experiment exp (its workload's task list). */
int msim_task_count(const msim_ctx *ctx, uint32_t exp, uint32_t *n_tasks);

/*
 * Start and finish tick of every task of experiment exp (the Schedule system,
 * Multiverse section 3.2), MSIM_NONE where the event has not happened yet;
 * arrays of msim_task_count entries, host memory, either may be NULL.
 * Synchronises hip_stream first.  Needs no recording; available for every
 * experiment after msim_bind.
 */
int msim_task_ticks(msim_ctx *ctx, uint32_t exp, void *hip_stream, uint32_t *start, uint32_t *finish);

/* Static description of the compiled batch, for callers and tests. */
typedef struct msim_info {
    uint32_t n_exp;
    uint32_t block_threads;      /* threads per workgroup (one workgroup simulates one experiment at a time) */
    uint32_t grid_blocks;        /* persistent workgroups launched by msim_run (0 before bind) */
    uint32_t lds_bytes;          /* dynamic LDS per workgroup (0: none; an experiment whose state stays in
                                    HBM may still copy its port table into it) */
    uint32_t n_lds_exp;          /* experiments whose state is worked on in LDS */
    uint32_t n_compact;          /* of those, experiments on the compact path (one thread per port) */
    uint32_t main_kernel;        /* kernel running most experiments: 0 msim_megakernel (general path);
                                    1..8 the compact path, msim_megakernel_c{8,16}{h,w}[_r1]: 8- or
                                    16-byte queue rows, 16- (h) or 32-bit (w) packet descriptors,
                                    _r1 when every link moves one packet per tick; kind =
                                    1 + (rows16 << 2 | desc32 << 1 | !r1) */
    uint32_t max_ports;          /* largest experiment: ports */
    uint64_t max_arena_bytes;    /* largest experiment: state bytes */
    uint64_t total_flows;        /* over the batch */
    uint64_t total_conns;
    uint64_t est_pkt_hops;       /* over the batch: sum of flow size x path links */
    uint64_t est_delivered;      /* over the batch: sum of flow sizes */
    uint64_t workspace_bytes;
} msim_info;

int msim_get_info(const msim_ctx *ctx, msim_info *info);

/* Message of the last error on this context (or, for ctx == NULL, of the last
 * failed msim_create on the calling thread). */
const char *msim_last_error(const msim_ctx *ctx);

/* Frees host-side state; the workspace stays the caller's. */
void msim_destroy(msim_ctx *ctx);

/* Measurement helper, not a step of the simulation: the LDS read bandwidth a
 * CU sustains, against which the runs that keep their state in LDS are
 * priced.  Launches `blocks` workgroups of 1,024 threads on hip_stream; each
 * fills 64 KiB of LDS, then every thread issues iters x 8 conflict-free
 * 16-byte LDS reads, so a launch reads blocks x 1,024 x iters x 128 bytes.
 * The caller times the launch (events on hip_stream).  dev_out: caller-owned
 * device memory of out_bytes >= blocks x 4,096 bytes; one 32-bit word per
 * thread is written to it (a fold of what the thread read).  Asynchronous.
 * MSIM_E_ARG for a NULL dev_out, too small an out_bytes, blocks == 0 or
 * > 2^20, or iters == 0; MSIM_E_HIP if the launch fails. */
int msim_lds_probe(void *dev_out, uint64_t out_bytes, uint32_t blocks, uint32_t iters, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* MSIM_H */
