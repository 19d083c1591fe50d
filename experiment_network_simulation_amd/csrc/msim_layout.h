/*
 * msim_layout.h -- private layout of the experiment-major state store shared by
 * the host compiler (msim_host.cpp) and the megakernel (msim_kernel.hip).
 *
 * Every experiment owns one contiguous "arena" in the workspace: a read-only
 * part (ports, connections, collective groups, host tables) followed by a
 * mutable part (virtual output queues, buffer pools, staging slots, connection
 * cursors).  The same byte offsets are valid whether the arena is used in HBM
 * or copied into a workgroup's LDS, so one kernel serves both placements.
 *
 * State owners of the general format (the pull discipline of Multiverse
 * section 4.2: each datum has one writer per phase, except for the
 * order-independent atomics named below and in msim_kernel.hip):
 *  - a switch ingress port q owns its buffer pool's descriptors and links
 *    (pdesc/pnxt), the tail side of its virtual output queues (tail, and the
 *    head byte of an empty queue) and its free-slot mask; it runs in phase A
 *    (arrivals);
 *  - a switch output port o owns the head side of the queues it drains
 *    (nslot), the in-flight and round-robin bytes of its output word and the
 *    staging slots of the ingress it feeds; it runs in phase D (grant, pop,
 *    transmit), returning each popped slot to its ingress's free mask and
 *    counting the pop in the word of the output feeding that ingress, both
 *    by atomic OR / add (several outputs may take from one ingress in a
 *    tick), and updates its own word with one atomic add;
 *  - a host owns its NIC (phase D), its deliveries and activations (phase A),
 *    the sender cursors of its outgoing connections and the receiver cursors of
 *    its incoming ones.
 */
#ifndef MSIM_LAYOUT_H
#define MSIM_LAYOUT_H

#include <stddef.h>
#include <stdint.h>

#define MSIM_NONE 0xFFFFFFFFu
/* ArenaHdr.cc: the experiment's congestion control (msim.h's MSIM_CC_* values) */
#define CC_DCTCP 1u
#define CC_DCQCN 2u
#define CC_HPCC 3u
#define MSIM_LAUNCH_TICKS (1u << 30)   /* most ticks one kernel launch simulates */

/* group kinds */
#define GK_RING_AR 1
#define GK_RING_AG 2     /* also the ring reduce-scatter: the same chunks along the same ring */
#define GK_BCAST 3
#define GK_XFLOW 4
#define GK_SEQ 5         /* send/recv unit task: one source, receivers in turn */
#define GK_TREE 6        /* binary-tree all-reduce, pipelined in chunks */

/* sender state of a connection (top two bits of ConnRW.s_pos) */
#define CS_WAIT 0u   /* previous flow just finished sending (or start): check at next phase A */
#define CS_IDLE 1u   /* waiting for its receive predecessor */
#define CS_ACTIVE 2u /* sending */
#define CS_DONE 3u   /* all flows sent */
#define CS_SHIFT 30
#define CS_POS_MASK 0x3FFFFFFFu

/* descriptor of a packet: connection << 4 | index of the next switch on its path;
 * in the general format bit 31 carries the ECN mark (connections < 2^27) */
#define DESC_SHIFT 4
#define DESC_HOP_MASK 0xFu
#define DESC_MARK 0x80000000u

struct PortRO {          /* 24 bytes */
    uint32_t peer;       /* port index at the far end of the cable */
    uint32_t base;       /* first port index of this node */
    uint32_t vbase;      /* first queue index of this node (switches) */
    uint32_t host;       /* host ports: host index; switch ports (general format): buffer pool
                            of the switch's port 0 (port k's pool is that + k) */
    uint8_t local, deg, rate, delay;
    uint8_t alive, is_host, peer_is_host, pad;
};

struct ConnRO {          /* 16 bytes */
    uint32_t route;      /* egress local port at switch i of the path in bits 4i..4i+3 */
    uint32_t grp;        /* collective group */
    uint32_t idx;        /* ring rank / broadcast hop-1 / explicit flow: packets */
    uint32_t lidx;       /* index among the source host's connections */
};

struct Grp {             /* 40 bytes */
    uint32_t kind;
    uint32_t N;          /* ring / tree members; broadcast: hops A; explicit: flow count;
                            send/recv: receivers */
    uint32_t S;          /* ring: steps per round; broadcast: partitions K; send/recv, tree: 1 */
    uint32_t R;          /* ring: rounds; tree: chunks */
    uint32_t p;          /* ring, tree: chunk packets; broadcast, send/recv: message packets */
    uint32_t X;          /* ring: packets in the last round; tree: in the last chunk;
                            send/recv: number of groups it gates */
    uint32_t fid_base;   /* first flow id */
    uint32_t conn_base;  /* first connection */
    uint32_t link;       /* ring: the send/recv group gating its first step, or MSIM_NONE;
                            send/recv: the first group it gates (they are consecutive) */
    uint32_t task;       /* the task that starts this group's collective, or MSIM_NONE */
};

/* task graph (general format only) */
#define TK_COMPUTE 0u
#define TK_INTRA 1u
#define TK_COLL 2u

struct TaskRO {          /* 24 bytes */
    uint32_t type;       /* TK_* */
    uint32_t dur;        /* compute / intra-server: duration in ticks (>= 1) */
    uint32_t pred_off, npred;  /* into the task predecessor list */
    uint32_t grp_first, ngrp;  /* collective task: its collective's groups */
};

struct TaskRW {          /* 16 bytes */
    uint32_t start, finish;    /* ticks, MSIM_NONE until known */
    uint32_t left;             /* collective task: flows not yet received */
    uint32_t pad;
};

struct HostRO {          /* 16 bytes */
    uint32_t port;
    uint32_t out_off;    /* into the host out-connection list */
    uint32_t n_out;
    uint32_t rdy_off;    /* first 32-bit word of the host's ready mask */
};

struct PortRW {          /* 16 bytes */
    uint32_t pad0;
    uint32_t pushed;     /* switch output under HPCC: packets sent on it (its telemetry) */
    uint32_t rr;         /* host NIC: round-robin pointer over its connections */
    uint32_t pad1;
};

struct ConnRW {          /* 16 bytes */
    uint32_t s_pos;      /* sender: flow position | state << 30 */
    uint32_t s_rem;      /* sender: packets left in the active flow */
    uint32_t r_pos;      /* receiver: flows fully received */
    uint32_t r_rem;      /* receiver: packets left in flow r_pos */
};

/* congestion control of a connection (general format, exp_cc = DCTCP) */
#define CC_NONE 0u
#define CC_DCTCP 1u
#define CWND_MAX_FP (65535u << 8)

struct CcRW {            /* 64 bytes: DCTCP */
    uint32_t cwnd;       /* window, 1/256 packet */
    uint32_t alpha;      /* 1/1024 */
    uint32_t sent, acked;/* packets over the connection */
    uint32_t wend;       /* acknowledged count that ends the current window */
    uint32_t wa, wm;     /* ACKs and marked ACKs in the window */
    uint32_t lat;        /* sum of the path's link delays: ACK delay */
    uint32_t aword;      /* the source host's ACK-pending word holding this connection's bit */
    uint32_t pad[7];
};

/* DCQCN (Zhu et al., SIGCOMM 2015) per connection, in the same 64-byte slot;
 * lat and aword where CcRW has them */
#define QCN_ONE 65536u          /* one packet per tick */
#define QCN_RMIN 64u
#define QCN_PERIOD 640u         /* rate-increase and alpha timers, ticks */
#define QCN_BYTES 2560u         /* packets between byte-counter events */
#define QCN_F 5u                /* stages of fast recovery */
#define QCN_AI 64u
#define QCN_HAI 160u
#define QCN_CNP_GAP 608u        /* ticks between a connection's CNPs */
struct QcnRW {
    uint32_t rc, rt;     /* current and target rate, 1/65536 packet per tick */
    uint32_t alpha;      /* 1/1024 */
    uint32_t tcnt, bcnt; /* timer and byte-counter stages */
    uint32_t bsent;      /* packets sent since the last byte-counter event */
    uint32_t last_cnp;   /* destination side: tick of the last CNP sent, or MSIM_NONE */
    uint32_t lat, aword;
    uint32_t next_inc, next_alpha;  /* next timer events */
    uint32_t pad0;
    uint64_t next_fp;    /* next send time, 1/65536 tick */
    uint32_t pad[2];
};
/* HPCC (Li et al., SIGCOMM 2019) per connection, in the same 64-byte slot;
 * sent, acked, lat and aword where CcRW has them.  Telemetry: per connection,
 * `slots` records of hx switches x 3 words (tick, egress packets sent,
 * backlog | rate << 24) from word 3 * hx * int_off of o_int, record seq %
 * slots for the packet with that sequence number; the last ACK's telemetry at
 * o_hl, 3 * hx words per connection */
#define HP_ETA 62259u           /* 0.95 in 1/65536 */
#define HP_MAX_STAGE 5u
#define HP_N 16u                /* flows expected to share a link, in W_AI */
struct HpRW {
    uint32_t w, wc;      /* window and reference window, 1/256 packet */
    uint32_t sent, acked;
    uint32_t U;          /* utilisation, 1/65536 */
    uint32_t stage;
    uint32_t hlast;      /* packets sent when Wc last changed */
    uint32_t lat, aword;
    uint32_t T;          /* base round trip 2 lat, ticks; the window cap in packets */
    uint32_t wai;        /* additive step, 1/256 packet */
    uint32_t have;       /* an ACK's telemetry has been recorded */
    uint32_t nsw;        /* switches on the path */
    uint32_t slots;      /* telemetry records (= T) */
    uint32_t int_off;    /* first record */
    uint32_t pad;
};
static_assert(sizeof(CcRW) == 64 && sizeof(QcnRW) == 64 && sizeof(HpRW) == 64, "congestion-control slots");
static_assert(offsetof(CcRW, sent) == offsetof(HpRW, sent) && offsetof(CcRW, acked) == offsetof(HpRW, acked) &&
              offsetof(CcRW, lat) == offsetof(HpRW, lat) && offsetof(CcRW, aword) == offsetof(HpRW, aword),
              "shared fields");
static_assert(offsetof(CcRW, lat) == offsetof(QcnRW, lat) && offsetof(CcRW, aword) == offsetof(QcnRW, aword),
              "shared fields");

struct HostRW {          /* 32 bytes */
    uint32_t pad0;
    uint32_t started;    /* first activation pass done */
    uint32_t left;       /* flows still to be received by this host */
    uint32_t pad;
    uint32_t pend[4];    /* MSIM_MAX_RATE */
};

/* Two arena formats.  Both start with {mode, bytes, rw_off, n_flows}.
 *  MODE_GENERAL: every datum in the arena (LDS or HBM placement), any thread
 *    count (threads stride over ports); no size limits beyond the ABI's.
 *  MODE_COMPACT: one thread per port; port-private state lives in registers
 *    during a run (saved in the arena between runs); the state other threads
 *    read is a compact image that is always copied into LDS. */
#define MODE_GENERAL 1u
#define MODE_COMPACT 2u

struct ArenaHdr {        /* general format header */
    uint32_t mode, bytes, rw_off, n_flows;
    uint32_t n_ports, n_hosts, n_conn, n_grp;
    uint32_t Q, W, R, n_voq;
    uint32_t o_port, o_conn, o_grp, o_hout, o_host;
    /* queue (ingress i, output o) of a switch: byte vbase + o * deg + i of
     * o_nslot (head slot, Q_EMPTY when empty) and o_tail (tail slot); the
     * ingress's free slots: four words at o_fmask + 32 * pool; o_ow[p]: output
     * p's word (packets in flight toward the far ingress, the packets taken
     * from that ingress during ticks of parity 0 and 1, a switch output's
     * round-robin pointer; one byte each); o_qlen[p] (congestion control):
     * packets queued for output p */
    uint32_t o_tail, o_nslot, o_fmask, o_ow, o_qlen;
    uint32_t o_pdesc, o_pnxt, o_pstate, o_scnt, o_sdesc, o_cstate, o_hstate, o_ready;
    uint32_t n_task, o_task, o_tpred, o_trw;
    /* congestion control: ACKs of connection c due at tick t are counted in the
     * 16-bit word o_ack[c * WA + t % WA] (ACKs | marked << 8), written by c's
     * destination host, read and cleared by its source at tick t, which finds
     * them through its ACK-pending masks o_ackm[(t % WA) * n_rdy + word] (one
     * bit per outgoing connection, the host's ready-mask layout, n_rdy words);
     * o_bl[o] is switch output o's backlog after the pops of the previous tick */
    uint32_t cc, ecn_k, WA, o_cc, o_ack, o_bl, o_ackm, n_rdy;
    /* packet spraying (lb = 1): descriptors are conn << sbits | sequence number;
     * o_spi[p] = node | (table row of the switch) << 16 | (fed from above) << 31;
     * o_cand[(row * n_hosts + dst) * 2 + down_only] = the switch's equal-cost
     * egress ports toward host dst (a 16-bit mask); ConnRO.route holds the
     * destination host; o_sseq / o_rnext: per connection, packets sent and
     * packets delivered in order; o_rbits: per connection, a bitmap of arrived
     * sequence numbers, words o_rwoff[c] .. o_rwoff[c+1]-1 */
    uint32_t lb, sbits, seed, o_spi, o_cand, o_sseq, o_rnext, o_rwoff, o_rbits;
    uint32_t o_hpc;      /* per host, one byte: connections whose flow finished sending last tick */
    /* split placement: [0, ro_hot) and [rw_off, rw_hot) hold everything the
     * switch phases and the host NICs touch each tick (ports, hosts, queues,
     * pools, staging, backlogs, host state); a workgroup that cannot hold the
     * whole arena in LDS copies these two ranges there, back to back, and
     * leaves the per-connection state in HBM; one that cannot hold these
     * either copies the port table alone (n_ports PortRO from o_port) */
    uint32_t ro_hot, rw_hot;
    /* HPCC (cc = 3): general-path descriptors are conn << cshift | telemetry
     * record << 4 | switches passed (cshift = DESC_SHIFT otherwise); hx
     * switches per telemetry record; o_hl, o_int as HpRW describes */
    uint32_t cshift, hx, o_hl, o_int;
};

/* ---- compact format ------------------------------------------------------
 * Thread slots: host ports 0..H-1, then switch ports from SB (H rounded up to a
 * wavefront); a switch's ports are consecutive and never straddle two
 * wavefronts, so everything a switch's ports exchange inside a tick stays in
 * one wavefront and a tick needs a single workgroup barrier.  A switch's
 * queue rows are rsz bytes (8 or 16): queue (i, o) of switch s is byte
 * vbase + o*rsz + i of the popper-major arrays and vbase + i*rsz + o of the
 * ingress-major ones. */

#define C_POS_MASK 0x3FFFu   /* CRW2.s_st: flow position (14 bits) | state << 14 */
#define C_STATE_SHIFT 14

struct ArenaHdr2 {       /* 144 bytes */
    uint32_t mode, bytes, rw_off, n_flows;
    uint32_t lds_bytes;  /* [0, lds_bytes) is the LDS image */
    uint32_t nt, H, SB;
    uint32_t Q, W, R, n_conn;
    uint32_t n_grp, rsz, dt, o_fmask;
    uint32_t o_arr, o_head, o_nslot, o_pdesc, o_pnxt, o_popped, o_elig, o_sdesc;
    uint32_t o_route, o_cgrp, o_lidx, o_crw, o_grp, o_hout;
    uint32_t o_port, o_priv;
    uint32_t flags, pad1[3];     /* AF_* */
};
#define AF_RINGS_ONLY 1u         /* every collective group is a ring */
/* Buffer pools are slot-major: slot s of the ingress on switch thread slot
 * SB + j lives at index s * (nt - SB) + j of pdesc / pnxt, so lanes touching
 * the same slot number of their own pools hit different LDS banks.
 * Staging (o_sdesc): for tick slot w and port slot p, RP
 * entries at (w * nt + p) * RP, entry m = descriptor + 1 of the m-th packet the
 * far output sent for that tick, 0 = empty; RP = the largest rate rounded up
 * to 1, 2 or 4. */
/* Queues: the byte of queue (i, o) in o_nslot is its head slot, Q_EMPTY when
 * the queue is empty (slots are < 64), and in o_arr its tail slot.  Each
 * switch ingress keeps its free buffer slots in a register; an output that
 * pops a slot returns it by an atomic OR into the ingress's word of o_fmask
 * (index slot - SB), which the ingress takes back when its register runs dry.
 * o_head and o_elig are unused (0). */
#define Q_EMPTY 0xFFu
/* popped, [2][nt]: [(t&1) * nt + slot] counts the pops from switch ingress
 * slot during tick t alone: the ingress zeroes it when the tick starts, the
 * outputs of its switch add to it, and the far output adds it to its own
 * running count during tick t+1. */

/* Collective group as the compact path reads it: the constant quotients of
 * the flow-size rules are precomputed, and pos / S is umulhi(pos << 8, mS),
 * exact for pos < 2^14 and S < 2^10. */
struct CGrp {            /* 48 bytes: three 16-byte loads */
    uint16_t kind, N;    /* ring / tree members; broadcast hops; send/recv receivers;
                            explicit: flow count (low 16 bits) */
    uint32_t S;          /* ring: steps per round; broadcast: partitions K; tree, send/recv: 1 */
    uint32_t R;          /* ring: rounds; tree: chunks */
    uint32_t p;          /* ring, tree: chunk packets; broadcast: packets / K; send/recv: message packets */
    uint32_t Xq;         /* ring: last-round packets / N; broadcast: packets mod K; tree: last chunk */
    uint32_t Xr;         /* ring: last-round packets mod N; send/recv: groups it gates */
    uint32_t fid_base, conn_base;
    uint32_t mS;         /* ceil(2^24 / S) */
    uint32_t link;       /* gated ring: its send/recv group; send/recv: first gated group; else MSIM_NONE */
    uint32_t pad[2];
};
static_assert(sizeof(CGrp) == 48, "CGrp is read as three 16-byte words");

struct CRW2 {            /* 8 bytes: compact connection cursors */
    uint16_t s_st, s_rem, r_pos, r_rem;
};

struct PortRO2 {         /* 16 bytes, one per thread slot (HBM) */
    uint32_t peer;       /* thread slot at the far end */
    uint32_t vbase;      /* switch: first queue byte; host: first out-connection list entry */
    uint16_t n_out;      /* host: outgoing connections */
    uint8_t local, deg, rate, delay, flags, pad;
};
#define PF_ALIVE 1u
#define PF_HOST 2u
#define PF_PEER_HOST 4u
#define PF_USED 8u

struct PortPriv {        /* 64 bytes: registers of a thread slot between runs */
    uint64_t freem;      /* switch ingress: free buffer slots */
    uint64_t ready;      /* host: connections with packets to send */
    uint32_t popped;     /* the far ingress's pops through the last tick */
    uint32_t pushed, rr, pcnt;
    uint32_t pend[4];
    uint32_t left, pad[3];
};

/* ---- ring format ----------------------------------------------------------
 * Experiments whose workload is rings only (at most 10 ranks each), every link
 * at rate 1, switches of at most 8 ports, buffers of at most 16 packets, paths
 * of at most 5 switches and at most 32 outgoing connections per host.  Thread
 * slots as in the compact format.  Everything lives in LDS during a run except
 * the per-thread registers (RingPriv, saved between runs) and the port table
 * (RingPort).
 *
 * Pairs.  In a ring every host that sends on connection (i -> i+1) of a
 * channel also receives on (i-1 -> i) of the same channel, and both flow
 * predecessors of its sends are local: the previous send on the same
 * connection and the previous receive on its partner.  A host's pair k joins
 * its k-th outgoing connection (index order: the NIC's round-robin order) with
 * that partner, so every flow event of a host touches one 16-byte record the
 * host alone owns.  Record (k, host h) sits at index k * SB + h.
 *
 * Descriptor of a packet (32 bits): bits 0..14 the egress port at each
 * remaining switch of its path, three bits each, the next switch's lowest;
 * bits 15..19 the pair index at the destination host; bit 20 set on the last
 * packet of a flow (a connection delivers in order, so its arrival completes
 * the flow); bits 21..30 the ring channel (group); bit 31 set (a staging word
 * of 0 means no packet).  A switch ingress stores it with its own hop shifted
 * out.
 *
 * Switch state (row of a port = switch * 8 + local port):
 *   pdesc[s * S + q], pnxt[s * S + q]  buffer slot s of ingress q (slot-major);
 *                      pnxt = Q_EMPTY after the last packet of a queue;
 *   head[row(o) * 8 + i]  head slot of queue (ingress i -> output o), written
 *                      by the ingress when it appends to an empty queue and by
 *                      the output when it pops;
 *   nzw[row(o)]        bit i: queue (ingress i -> output o) holds a packet; set
 *                      by the ingress (LDS atomic OR: several ingresses of a
 *                      switch may set bits of one word in one instruction),
 *                      cleared by the output when it pops the last packet;
 *   fw[t & 1][q]       what the outputs of its switch took from ingress q at
 *                      tick t: bit s = buffer slot s freed, bit 16 + o = queue
 *                      (q -> o) emptied (LDS atomic OR).  Read at tick t + 1 by
 *                      the ingress, which folds it into its registers, and by
 *                      the port that feeds q, which counts the pops for its
 *                      credit; cleared by the ingress at tick t + 2 before its
 *                      outputs write it again.  Each half holds S + 1 words;
 *                      word S stays 0 (the word a port without a far buffer
 *                      reads).
 * Staging: sdesc[(t mod W) * NS + stg(slot)] = descriptor of the packet
 * reaching that port at tick t, 0 for none, rewritten by its feeder every
 * tick; NS = nt rounded up to 64.  stg permutes the slots so that the 64
 * lanes of every wavefront read 64 different LDS banks (their own words) and
 * write 64 different banks (their far ends' words): a colouring with 64
 * colours (stg mod 64) of the edges of the bipartite multigraph that joins,
 * for every port slot, its wavefront as reader and its far end's wavefront as
 * writer, which exists since no wavefront has more than 64 lanes (Konig's
 * edge-colouring theorem); slots of one colour take stg = colour + 64 k.
 * Digest queue: dq[host * RING_DQ + k], the (flow << 32 | RD) words a host
 * has received but not yet mixed into its digest; a wavefront mixes all its
 * hosts' queues together once one of them is full, and at the end of a run. */
#define MODE_RING 3u
#define RING_MAX_DEG 8u
#define RING_MAX_Q 16u
#define RING_MAX_PAIRS 32u
#define RING_MAX_HOPS 5u
#define RING_MAX_N 10u
#define RD_ROUTE_MASK 0x7FFFu
#define RD_PAIR_SHIFT 15
#define RD_LAST 0x100000u
#define RD_GRP_SHIFT 21
#define RD_VALID 0x80000000u
#define RING_MAX_GRP 1024u
#define RING_DQ 4u

struct ArenaHdr3 {       /* 96 bytes */
    uint32_t mode, bytes, rw_off, n_flows;
    uint32_t lds_bytes, nt, H, SB;
    uint32_t Q, W, n_grp, n_sw;
    uint32_t o_grp, o_pair, o_pdesc, o_pnxt;
    uint32_t o_head, o_nzw, o_fw, o_dq;
    uint32_t o_sdesc, o_port, o_priv, pad;
};

struct RGrp {            /* 32 bytes: one ring channel */
    uint32_t fid_base;   /* flow id of (round 0, step 0, rank 0) */
    uint32_t N, S;       /* ranks; steps per round */
    uint32_t RS;         /* flows per connection: rounds x steps */
    uint32_t p;          /* packets per chunk of a full round */
    uint32_t Xq;         /* last round of X packets: chunk k holds Xq + [k < X mod N] */
    uint32_t T;          /* bit j, j < 3N: chunk j mod N of the last round holds Xq + 1 */
    uint32_t mS;         /* ceil(2^24 / S): pos / S = umulhi(pos << 8, mS) for pos < 2^14 */
};

struct RPair {           /* 16 bytes */
    uint32_t snd;        /* packets left in the active flow | position << 16 | state << 30 (CS_*) */
    uint32_t rcv;        /* flows received over the partner connection */
    uint32_t desc;       /* descriptor of the outgoing connection's packets at the first switch */
    uint32_t gi;         /* group | rank of this host << 10 | rank of its predecessor << 20 */
};

struct RingPort {        /* 16 bytes, one per thread slot (HBM) */
    uint32_t peer;       /* thread slot at the far end */
    uint32_t row;        /* switch: its switch's first row (switch * 8); host: outgoing connections */
    uint8_t flags, local, deg, delay;
    uint16_t stg;        /* this slot's staging word within a tick slot of the staging ring */
    uint16_t pstg;       /* ... and the far end's, where this slot's output stages its packet */
};

struct RingPriv {        /* 32 bytes: registers of a thread slot between runs */
    uint32_t pushed, rr;
    uint32_t mask;       /* switch: free buffer slots; host: pairs ready to send */
    uint32_t tails;      /* switch: tail slot of each of its queues (4 bits each); host: flows left to receive */
    uint32_t ne;         /* switch: bit o = queue toward o not empty */
    uint32_t seen;       /* packets forwarded out of the far buffer, as counted from its fw words */
    uint32_t pad[2];
};
static_assert(sizeof(RGrp) == 32 && sizeof(RPair) == 16 && sizeof(RingPort) == 16 && sizeof(RingPriv) == 32,
              "ring records");

/* per-experiment progress and totals (workspace, outside the arena) */
struct ExpState {        /* 64 bytes */
    uint32_t status;     /* MSIM_EXP_* */
    uint32_t t_now;      /* next tick to simulate */
    uint32_t t_out;      /* reported tick */
    uint32_t t_max;      /* largest RD so far */
    uint64_t pkt_hops, delivered, digest;
    uint32_t last_tx1;   /* 1 + last tick with a transmission (0: none) */
    uint32_t last_act1;  /* 1 + last tick with an activation (0: none) */
    uint32_t max_arr;    /* largest arrival tick of any packet sent */
    uint32_t fault;      /* nonzero: an internal invariant broke (status MSIM_EXP_FAULT) */
    uint32_t pad[2];
};

/* workspace header */
#define MSIM_KINDS 15
#define KIND_GENERAL_TASKS 9   /* the general path with a task graph */
#define KIND_GENERAL_CC 10     /* the general path with congestion control (and tasks, if any) */
#define KIND_COMPACT_X8 11     /* compact, 8-byte rows, rate 1, with trees / send-recv / gates */
#define KIND_COMPACT_X16 12    /* compact, 16-byte rows, a faster link, with trees / send-recv / gates */
#define KIND_GENERAL_SPRAY 13  /* the general path with packet spraying (and tasks, if any) */
#define COMPACT_X_THREADS 768  /* launch bound of the two kinds above */
#define KIND_RING 14           /* the ring format */

struct WsHdr {
    uint32_t claim[MSIM_KINDS]; /* experiment queue counters of a run, one per kernel kind */
    uint32_t n_exp;
    uint32_t pad[64 - MSIM_KINDS - 1];
};
static_assert(sizeof(WsHdr) == 256, "the workspace's first 256 bytes");

/* msim_run_noalloc: experiment queue counters, one per kernel launch of a
 * call, in a static device array of this many words instead of the workspace */
#define MSIM_SCRATCH_WORDS 64   /* msim.h's MSIM_NOALLOC_LAUNCHES */

struct KParams {
    uint8_t *ws;
    uint32_t *claim;     /* this launch's experiment queue counter, zero when the launch starts */
    uint64_t o_state, o_arena_off, o_order, o_rec_off, o_pristine, o_rw_off;
    uint32_t n_exp;
    uint32_t max_ticks;
    uint32_t lds_bytes;  /* dynamic LDS available to an arena (0: HBM only) */
    uint32_t order_base; /* this launch's experiments: order[order_base .. order_base + n_run) */
    uint32_t n_run;
    uint32_t pad;
};

#endif
