/*
 * purlin.h - C ABI of the Purlin collective hot path on one gfx950 GPU.
 *
 * Source of the semantics: "Purlin: Separating Orchestration from the
 * Datapath of Collectives" (arXiv 2609.36954).
 *   - A collective is specified by two layout namings (inputs, outputs) and an
 *     operation, copy or reduction (abstract).
 *   - Layouts: ReduceScatter combines partition k of every input into y_k at
 *     rank k; AllGather gives each rank all of y_0 .. y_{P-1}, ordered by rank;
 *     AllToAll gives rank j partition j of every source (Figure 4 caption).
 *   - AllReduce is ReduceScatter and AllGather composed chunk by chunk
 *     (Figure 6 caption).
 *   - (V) variants have variable partition sizes (Table 2, Figure 16).
 *   - Coordination is derived from the specification by the SNAC protocol
 *     (Stage, Notify, And Consume; abstract), the bytes are moved by the Atom
 *     copy and reduce primitives (abstract), and in the zero-staging variant
 *     (Purlin-ZS) consumers read the inputs directly, with no staging step
 *     (Figure 10 caption).
 *
 * The P "ranks" are P buffer sets in the memory of the one current HIP
 * device: each launch performs the share of every rank.  All pointers in
 * purlin_layout are device pointers owned by the caller; nothing here takes
 * ownership of them, frees them or keeps them after the call returns.
 *
 * Streams.  Every call is enqueued on the caller's stream and returns
 * without synchronizing the device or the stream.  Library workspace (flag
 * block, staging rings, MoE table) belongs to a stream: a call allocates it
 * the first time that stream needs it, and grows it with a new allocation
 * cleared in stream order (the old one stays allocated until
 * purlin_release), so no call waits for other work.  Calls on one stream run
 * in stream order; calls on different streams share no workspace and never
 * wait for each other, so they may run concurrently.  The zero-staging
 * collectives without the handshake (the default) use no workspace at all.
 *
 * HIP graphs.  Calls may be captured into a HIP graph and replayed any
 * number of times: launch epochs are kept in device memory, so every replay
 * gets a fresh one, and nothing the library enqueues is a memset or a copy.
 * A captured call must not need new workspace: make the same call (or a
 * larger one) on the capturing stream once before capture, else it returns
 * PURLIN_ERR_UNSUPPORTED.  A replayed graph uses the workspace of the stream
 * it was captured on; do not run it concurrently with calls on that stream.
 * Workspace is keyed by the stream handle: a stream destroyed while its work
 * is still running must not be replaced by a new one with the same handle.
 *
 * Host threads.  Any thread may call any function: the library serializes
 * its host bookkeeping (workspace, plan cache, policy) under one lock, and
 * the launches themselves stay asynchronous.  The policy is process-wide;
 * purlin_last_launch reports the calling thread's most recent launch.  Do
 * not call purlin_release while another thread's work may still be using
 * the workspace it frees.
 */
#ifndef PURLIN_H_
#define PURLIN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

#define PURLIN_MAX_RANKS 8

#ifndef PURLIN_API
#define PURLIN_API __attribute__((visibility("default")))
#endif

typedef enum {
  PURLIN_OK = 0,
  PURLIN_ERR_INVALID_ARG = 1, /* bad pointer, P, count, alignment, overlap */
  PURLIN_ERR_UNSUPPORTED = 2, /* the (naming, naming, op) triple is not a collective, or
                                 the call would need new workspace during graph capture */
  PURLIN_ERR_NO_MEMORY = 3,   /* workspace allocation failed */
  PURLIN_ERR_HIP = 4,         /* a HIP call or kernel launch failed */
  PURLIN_ERR_TIMEOUT = 5,     /* a bounded device wait expired (see purlin_check) */
  PURLIN_ERR_PROTOCOL = 6     /* the protocol-checking build saw a flag, credit or staging-slot
                                 header other than the protocol allows (see purlin_check) */
} purlin_status;

typedef enum { PURLIN_OP_COPY = 0, PURLIN_OP_SUM = 1 } purlin_op;

/* Element type.  SUM widens each element exactly to fp32, adds in fp32 in
 * ascending source rank, and rounds once to the output type (bf16: round to
 * nearest even).  COPY moves bytes and only uses the element size. */
typedef enum { PURLIN_F32 = 0, PURLIN_BF16 = 1 } purlin_dtype;

/* How a rank's buffer is split into partitions, and each partition's name
 * (r = the buffer's rank, q = the partition index). */
typedef enum {
  PURLIN_NAME_WHOLE = 0,         /* 1 partition,  name ()     */
  PURLIN_NAME_BY_RANK = 1,       /* 1 partition,  name (r)    */
  PURLIN_NAME_BY_INDEX = 2,      /* P partitions, name (q)    */
  PURLIN_NAME_BY_RANK_INDEX = 3, /* P partitions, name (r, q) */
  PURLIN_NAME_BY_INDEX_RANK = 4  /* P partitions, name (q, r) */
} purlin_naming;

typedef struct {
  purlin_naming naming;
  void *const *bufs; /* P device pointers, one buffer per rank; caller-owned.
                        A buffer holding no element of the collective may be NULL. */
} purlin_layout;

typedef enum {
  PURLIN_STAGING_AUTO = 0,  /* policy table decides */
  PURLIN_STAGING_ZS = 1,    /* zero staging: consumers read the inputs directly */
  PURLIN_STAGING_STAGED = 2 /* producers stage chunks in a ring, notify, consumers consume */
} purlin_staging;

/* Datapath of copy collectives (copy engines: the Figure 10 caption's
 * AllGather on the copy engine, without a kernel of its own, and the Figure 3
 * caption's point that copies need not occupy compute units). */
typedef enum {
  PURLIN_ENGINE_AUTO = 0,   /* shader kernels (the Atom) */
  PURLIN_ENGINE_SHADER = 1, /* shader kernels (the Atom) */
  PURLIN_ENGINE_COPY = 2    /* COPY collectives as stream-ordered transfers on the DMA copy
                               engines (hipMemcpyDeviceToDeviceNoCU), one per (output
                               partition, destination rank): no kernel, no compute unit.
                               SUM collectives still run on the shader kernels. */
} purlin_engine;

/* Execution policy (Figure 1 caption: policies chosen with the hardware in
 * mind decide how a collective runs).
 * A zero field means "automatic".  It never changes a result, only speed. */
typedef struct {
  int64_t chunk_bytes;   /* bytes per work chunk / staging slot; multiple of 4096 */
  int32_t depth;         /* staging slots per channel, 1..8 (staged only) */
  int32_t wgs_per_rank;  /* workgroups per rank; grid = P * wgs_per_rank */
  int32_t zero_staging;  /* purlin_staging */
  int32_t sync;          /* entry/exit notify (the per-rank handshake): 0 auto (off: calls
                            on one stream are ordered by the stream), 1 on, 2 off */
  int64_t watchdog_ns;   /* bound of every device spin wait */
  int32_t test_withhold; /* test only: k > 0 withholds the k-th ready notify
                            of staging channel 0, to exercise the watchdog */
  int32_t engine;        /* purlin_engine */
} purlin_policy;

/* One (output partition, matching input partition) pair of a plan. */
typedef struct {
  int32_t src_rank, dst_rank;
  int64_t src_off, dst_off, len; /* elements */
} purlin_segment;

/* What the calling thread's most recent successful call launched
 * (measurement only). */
typedef struct {
  int32_t grid;          /* workgroups launched */
  int32_t threads;       /* threads per workgroup */
  int32_t zero_staging;  /* 1 if the ZS kernel ran, 0 if the staged one */
  int32_t depth;         /* staging depth used (staged) */
  int64_t chunk_bytes;   /* chunk size used */
  int64_t tiles;         /* work chunks in the launch */
  int64_t bytes_min;     /* compulsory HBM bytes: inputs read once + outputs written once */
  int32_t njobs;
  int32_t sync;
  int32_t rows;          /* 1 if the kernel with the realigning row bodies ran (some source
                            off its destinations' 16-byte phase), 0 if the aligned-only one */
  int32_t unit;          /* purlin_ulysses: bytes each lane access moved (16, 8, 4 or 2);
                            0 for the other calls */
  int32_t one;           /* zero-staging launch: 1 if the build for single-destination jobs
                            ran (no broadcast in the launch), 0 otherwise */
  int32_t plain_stores;  /* 1 if the build with plain (not nontemporal) body stores ran:
                            copy broadcasts of 16 MiB of jobs or more, Ulysses exchanges of
                            at most 128 MiB each way */
  int32_t engine_copies; /* copy-engine transfers enqueued (PURLIN_ENGINE_COPY; grid is then
                            0: no kernel ran), 0 for kernel launches */
  int32_t shift_stores;  /* zero staging: jobs whose sources share a 16-byte phase off
                            their destination's took source-aligned units (reductions):
                            1 with misaligned stores, 2 shifted into aligned stores
                            across carried rows (32 MiB of jobs or more) */
  int32_t unaligned_loads; /* zero staging: 1 if jobs with a source off their destinations'
                              phase took destination-aligned units and misaligned loads
                              (copy broadcasts of 32 MiB of jobs or more) */
  int32_t device_stores; /* zero staging: 1 if broadcast jobs were stored at device scope
                            (written through the L2) */
  int32_t unroll;        /* collective kernels: 16-byte units each lane keeps in flight per
                            source (copies 4 / 8 / 16, sums 1 / 2 / 4); 0 otherwise */
} purlin_launch_info;

/*
 * Run one collective over P ranks, asynchronously on `stream`.
 *
 * Output partition (j, s) receives `op` applied to every input partition
 * (i, q) whose name equals its own, in ascending i: COPY needs exactly one
 * such partition, SUM at least one.  The seven collectives:
 *
 *   collective        in naming      out naming     op    counts
 *   AllReduce         WHOLE          WHOLE          SUM   [N]
 *   ReduceScatter(V)  BY_INDEX       BY_RANK        SUM   [c_0 .. c_{P-1}] (y_k has c_k)
 *   AllGather(V)      BY_RANK        BY_INDEX       COPY  [c_0 .. c_{P-1}] (rank k sends c_k)
 *   AllToAll(V)       BY_RANK_INDEX  BY_INDEX_RANK  COPY  [P*P], counts[i*P+j] = size of
 *                                                          partition j of rank i = slot i of rank j
 *
 * counts: one element count per name (names (a, b) are numbered a*P + b);
 *   so it holds 1 entry for WHOLE, P for BY_RANK / BY_INDEX and P*P for the
 *   pair namings.  A collective is "V" exactly when its counts differ.
 * displs: NULL for partitions packed in index order, or 2 * len(counts)
 *   element offsets: the input offsets then the output offsets, each indexed
 *   by name like counts, into the buffer of the rank holding that name
 *   (BY_INDEX and WHOLE offsets are shared by every rank).  Output elements
 *   outside every partition are never written.
 *
 * Requirements (else PURLIN_ERR_INVALID_ARG, checked before any HIP call):
 *   1 <= P <= 8; non-NULL layouts and counts; counts and displs >= 0; every
 *   buffer that holds an element non-NULL and aligned to the element size;
 *   output partitions disjoint; no input byte overlaps an output byte.
 * Other (naming, naming, op) triples return PURLIN_ERR_UNSUPPORTED, and so
 * does a plan of more than 64 jobs (a sum of P partitions broadcast to every
 * rank, by_index -> by_index, whose output buffers are not all congruent
 * modulo 16 bytes), also checked before any HIP call.
 *
 * The call enqueues one kernel and returns; it never synchronizes.  Inputs
 * must stay valid and outputs untouched until the stream reaches that point.
 * The staged variant's workgroups wait for each other; they are numbered so
 * that every job's producers come before its consumers and the jobs before
 * the one being started are wholly resident, so a kernel beside it on
 * another stream that finishes on its own delays it but cannot block it.
 * Two staged launches on different streams can block each other when
 * together they need more workgroups than the device holds and a producer
 * waits for a slot's credits (a lane with more chunks than ring slots): the
 * watchdog then ends both with PURLIN_ERR_TIMEOUT.  Keep staged launches on
 * one stream, or give the policy a depth of at least the chunks per lane.
 * A device-side watchdog expiry is reported by purlin_check.
 */
PURLIN_API purlin_status purlin_collective(const purlin_layout *in, const purlin_layout *out,
                                purlin_op op, purlin_dtype dtype, int P,
                                const int64_t *counts, const int64_t *displs,
                                hipStream_t stream);

/*
 * purlin_collective for callers that cannot allocate device memory on the
 * call path: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, semantics and synchronous errors
 * as purlin_collective; it calls no hipMalloc, hipFree or other allocating
 * routine.  Instead of its stream's workspace it uses one fixed array in
 * device memory per GPU, held from the first call on that GPU until the
 * process ends: a 8 KiB flag block, 256 KiB of staging slot flags (1024
 * slots) and 32 MiB of staging rings.  The first call on a device looks up
 * the array's address (make it outside graph capture).  A staged plan is
 * shrunk to fit the array (depth down to 2, fewer pipelines, chunks down to
 * 4 KiB, as far as the policy leaves them open); when the policy fixes a
 * plan larger than the array the call returns PURLIN_ERR_NO_MEMORY and
 * enqueues nothing.  Zero staging without the handshake uses none of the
 * array.  Every call on a GPU shares that GPU's array: calls whose
 * execution overlaps on one GPU (on different streams, or a graph replayed
 * beside an eager call) race and are not supported; calls in one stream's
 * order are.  A device-side timeout of such a call is reported by
 * purlin_check on any stream of that device.
 */
PURLIN_API purlin_status purlin_collective_noalloc(const purlin_layout *in,
                                                   const purlin_layout *out, purlin_op op,
                                                   purlin_dtype dtype, int P,
                                                   const int64_t *counts, const int64_t *displs,
                                                   hipStream_t stream);

/* Synchronize `stream`, then read and clear that stream's device status
 * word (current device): PURLIN_ERR_TIMEOUT if any wait of a call on the
 * stream expired since the last check, else PURLIN_ERR_PROTOCOL if the
 * library was built with PURLIN_DEBUG_PROTOCOL and one of its checks failed
 * (a staged flag or credit past the value the protocol allows at that
 * point, or a staging slot whose header or canary is not the one its
 * producer wrote for that chunk), else PURLIN_ERR_INVALID_ARG if a
 * device-side argument check failed (MoE indices), PURLIN_ERR_HIP if the
 * synchronization failed, else PURLIN_OK.  This call synchronizes. */
PURLIN_API purlin_status purlin_check(hipStream_t stream);

/* Replace the policy (NULL restores the defaults).  Environment variables
 * PURLIN_CHUNK_BYTES, PURLIN_DEPTH, PURLIN_WGS_PER_RANK, PURLIN_ZS (0/1),
 * PURLIN_SYNC (0/1), PURLIN_WATCHDOG_NS and PURLIN_ENGINE (purlin_engine)
 * override the defaults only.  INVALID_ARG for out-of-range fields.  Takes
 * effect on the next call.
 *
 * Datapath switches, read at every call, for measurement (each selects
 * between forms that give identical results; unset = the measured default):
 * PURLIN_SHIFT_STORES (0/1/2: sums whose sources share a 16-byte phase off
 * their destination's take the row body / source-aligned units with
 * misaligned stores / the same units shifted into aligned stores across
 * rows each wavefront carries),
 * PURLIN_UNALIGNED_LOADS (0/1: copies off their destination's phase take
 * destination-aligned units with misaligned loads), PURLIN_BCAST_PLAIN (0/1:
 * plain stores for large copy broadcasts), PURLIN_NT (0/1: nontemporal
 * loads and stores), PURLIN_NT_ANY_PHASE (0/1: nontemporal loads also for
 * sources off their destination's 128-byte phase), PURLIN_UNROLL (0, 1, 2:
 * units per lane in flight, copies 4 / 8 / 16, sums 1 / 2 / 4), PURLIN_LDS
 * (0/1: the LDS-staged aligned body), PURLIN_OWNER_TEAM (1-8: owner
 * workgroups per staged reduction lane), PURLIN_MID_CHUNKS (0/1: the
 * mid-size grid and chunk rules of the policy table, and AllToAll's one
 * workgroup per CU from 1 GiB of jobs), PURLIN_DEVICE_STORES (0/1:
 * broadcast stores at device scope, written through the L2),
 * PURLIN_LARGE_BCAST (0/1: the grid and chunk of large aligned copy
 * broadcasts). */
PURLIN_API purlin_status purlin_set_policy(const purlin_policy *p);

/* The policy in force (defaults, environment, then purlin_set_policy). */
PURLIN_API purlin_status purlin_get_policy(purlin_policy *p);

/* Test/debug: the plan of a collective without running it (no HIP call).
 * Writes up to *n_segs segments to segs (which may be NULL) and sets *n_segs
 * to the number the plan has.  Same argument rules as purlin_collective. */
PURLIN_API purlin_status purlin_plan_describe(const purlin_layout *in, const purlin_layout *out,
                                   purlin_op op, purlin_dtype dtype, int P,
                                   const int64_t *counts, const int64_t *displs,
                                   purlin_segment *segs, int64_t *n_segs);

/*
 * MoE dispatch (expert parallelism; the MoE call sites of AllToAll in Table 2
 * of the Purlin pages) with the token permutation folded into the exchange:
 * an AllToAllV whose send rows are read by token index.
 *
 *   x[i]       rank i's token rows, x_rows[i] rows of row_bytes bytes (input)
 *   idx[i]     device int32 array: rank i's entries, the row indices to send,
 *              grouped by destination rank: counts[i*P + j] entries for rank j,
 *              group j after group j-1 (input)
 *   counts     host, P*P row counts, [i*P + j] = rows from rank i to rank j
 *   x_rows     host, P row counts of the x[i]
 *   y[j]       rank j's received rows, sum_i counts[i*P + j] rows: for i
 *              ascending, rows x[i][idx[i][group j]] in entry order (output)
 *
 * unique != 0 promises one row per (token, destination rank) (the
 * deduplicated routing): each token row is then read once and written to
 * every rank it goes to, through a table of sum(x_rows) * P 8-byte words the
 * library keeps per stream (as purlin_moe_combine); a token twice in one
 * group is then reported.  unique == 0 gathers row by row and allows repeats.
 *
 * Rows are moved as bytes (row_bytes even and at most 1 GiB, buffers 2-byte
 * aligned; 16-byte alignment of every buffer and of row_bytes takes the
 * faster kernels, and is needed for the by-token path).  Ownership as
 * purlin_collective.
 * Synchronous errors: INVALID_ARG for P outside [1, 8], a NULL array or
 * buffer that holds data, a negative count, odd row_bytes or one above
 * 1 GiB, entries for a
 * rank with no rows, an output overlapping an input or another output.
 * Asynchronous: an index outside [0, x_rows[i]) skips its row and makes the
 * next purlin_check return INVALID_ARG.  Asynchronous on `stream`.
 */
PURLIN_API purlin_status purlin_moe_dispatch(void *const *x, void *const *y, int P,
                                             int64_t row_bytes, const int32_t *const *idx,
                                             const int64_t *counts, const int64_t *x_rows,
                                             int unique, hipStream_t stream);

/*
 * MoE combine: the reverse exchange of purlin_moe_dispatch with a weighted
 * sum per token.  y[j] holds rank j's rows in dispatch order (bf16, input);
 * w[i] is a device float array, one weight per entry of idx[i] (input);
 * out[i] gets x_rows[i] bf16 rows:
 *
 *   out[i][t] = RNE_bf16( fp32 left fold from +0, over the entries (j, k)
 *               of idx[i] with idx[i][group j + k] == t in ascending j then
 *               k, of  w[i][entry] * y[j][row of (i, j) + k] )
 *
 * each product rounded to fp32 before its add.  A token routed nowhere gets
 * +0.  One row per (token, destination rank): a token twice in one group is
 * reported.  row_bytes a multiple of 16 and every buffer 16-byte aligned.
 * The library keeps a table of sum(x_rows) * P 8-byte words per stream
 * (allocated on the first call on the stream that needs it, freed by
 * purlin_release).  Errors as
 * purlin_moe_dispatch, plus INVALID_ARG for misalignment or a NULL weight
 * array that holds entries; a duplicate token in a group also makes the
 * next purlin_check return INVALID_ARG (that token's row is unspecified).
 */
PURLIN_API purlin_status purlin_moe_combine(void *const *y, void *const *out, int P,
                                            int64_t row_bytes, const int32_t *const *idx,
                                            const float *const *w, const int64_t *counts,
                                            const int64_t *x_rows, hipStream_t stream);

/*
 * Ulysses sequence-parallel AllToAll (Purlin pages, Table 2: in the diffusion
 * workload an AllToAll moves activations between a sequence-sharded and a
 * head-sharded layout).  P ranks, `heads` attention heads (a multiple of P), each
 * head `head_bytes` bytes per token (head dimension x element size; even),
 * seq[i] >= 0 tokens on rank i (host array of P), S = sum of seq.  Layouts,
 * row-major, tokens of rank 0 first in the head layout:
 *
 *   sequence layout  rank i:  [seq[i], heads, head_bytes]
 *   head layout      rank j:  [S, heads / P, head_bytes]   (head group j)
 *
 * to_sequence = 0: in = sequence layout, out = head layout,
 *   out[j][off_i + s][h] = in[i][s][j * heads / P + h],  off_i = seq[0] + ... + seq[i-1];
 * to_sequence = 1: the inverse (in = head layout, out = sequence layout).
 * Bytes are copied as they are (any element type).  Several tensors that
 * share a token axis, laid out [tokens, n, heads, head_bytes] (query, key and
 * value of a fused projection), exchange in one call with seq[i] * n as the
 * token counts.  in and out are host arrays of P device pointers (a pointer
 * may be NULL only where its buffer is empty); every out buffer is disjoint
 * from every in buffer.  Returns INVALID_ARG for a bad count, size,
 * alignment (odd addresses) or overlap, HIP for a launch failure.
 * Asynchronous on `stream`; runs the entry / exit handshake when the policy
 * asks for it, like purlin_collective.
 */
PURLIN_API purlin_status purlin_ulysses(void *const *in, void *const *out, int P,
                                        const int64_t *seq, int64_t heads, int64_t head_bytes,
                                        int to_sequence, hipStream_t stream);

/* Measurement: the launch shape of the calling thread's most recent
 * successful call. */
PURLIN_API purlin_status purlin_last_launch(purlin_launch_info *info);

/* Measurement: a plain 128-bit streaming copy of `bytes` bytes (both
 * pointers 16-byte aligned, bytes a multiple of 16), the calibration and
 * ceiling kernel for HBM counters.  Asynchronous on `stream`. */
PURLIN_API purlin_status purlin_stream_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream);

/* Measurement: the bare memory pattern of a collective, as a ceiling.  Each
 * 16-byte unit u < bytes/16 is read from n_src sources (added as integers)
 * and the result written to n_dst destinations, at the same offset in every
 * buffer; n_src and n_dst in {0, 1, 8}, not both 0 (n_src 0: write-only, a
 * pattern of the unit index; n_dst 0: read-only), all pointers 16-byte
 * aligned and every destination disjoint from every source.  `grid`
 * workgroups (0: four per CU, at most 65536) walk tiles of tile_bytes (0:
 * 16 KiB; a multiple of 16, below 4 GiB) in grid-stride order, `unroll`
 * 16-byte units per lane in flight (0: 4; else 2, 4 or 8; eight sources
 * take at most 4), with no planning or flags, as the collectives walk
 * theirs.  access bit 0: nontemporal loads, bit 1: nontemporal stores, bit
 * 2: device-scope stores (written through the L2; bit 1 is then ignored).
 * INVALID_ARG otherwise.  Asynchronous on `stream`. */
PURLIN_API purlin_status purlin_stream_pattern(const void *const *srcs, int n_src,
                                               void *const *dsts, int n_dst, int64_t bytes,
                                               int grid, int64_t tile_bytes, int unroll,
                                               int access, hipStream_t stream);

/* Static text for a status code. */
PURLIN_API const char *purlin_strerror(purlin_status s);

/* Synchronize every device the library has used and free the library-owned
 * workspace of every stream (flags, staging rings, MoE tables, outgrown
 * buffers).  The next call that needs workspace allocates it again.  Graphs
 * captured before must not be replayed afterwards. */
PURLIN_API void purlin_release(void);

#ifdef __cplusplus
}
#endif

#endif /* PURLIN_H_ */
