/*
 * sparse_topk.h -- C ABI of the indexer top-k selection library for MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * The lmsys.org page "Serving GLM5.2 NVFP4 Agentic Workload with SGLang",
 * section "Kernel Optimization / TopK-V2" (text and the captions of Figures 2,
 * 3 and 4), describes the DSA indexer's top-k step: each query row holds FP32
 * scores over historical KV positions; the kernel returns exactly k of those
 * positions (runtime k up to 2048), decided exactly at the FP32 boundary with
 * an exact tie-break, and translates every selected logical position into a
 * physical indexer-KV-cache slot through the paged block table, in the same
 * kernel. A planning kernel, run once per forward and reused across indexer
 * layers, turns the batch's length distribution into a work list.
 *
 * For row r with n = lengths[r] valid scores the selected set is
 *     the first min(k, n) positions of [0, n) ordered by
 *     (score descending, position ascending),
 * i.e. ties at equal score go to the lower logical position (the page does not
 * print the tie rule; this is the reading the library implements). -0.0 and
 * +0.0 are equal scores; -inf is an ordinary lowest score. Positions >= n are
 * never read as candidates, whatever they hold.
 * Selected position i maps to slot  block_table[r * bt_row_stride + i / page_size]
 *                                    * page_size + i % page_size.
 *
 * Output of a row: entries [0, min(k, n)) hold the selected positions' slots in
 * UNSPECIFIED order (the page treats top-k as selection, not sorting); entries
 * [min(k, n), k) hold -1. When out_indices is given, out_indices[r][j] is the
 * logical position whose slot is out_slots[r][j].
 *
 * Memory and threading
 * --------------------
 * All data pointers are DEVICE pointers unless a parameter says "host". All
 * work is enqueued asynchronously on `stream` (a hipStream_t passed as void*;
 * NULL means the default stream). The caller owns every buffer. topk_plan and
 * topk_select_paged never allocate, free or synchronise, so both may be
 * captured into a HIP graph. A workspace must not be used by two calls that
 * can run at the same time.
 *
 * Errors
 * ------
 * Host-checkable argument errors are returned synchronously and nothing is
 * enqueued. Violations of the device-data contract below cannot be checked
 * without a synchronisation; results are then undefined, and a device status
 * word in the workspace may record them (topk_read_status):
 *   0 <= lengths[r] <= max_len and <= score_row_stride;
 *   no NaN among the valid scores;
 *   the block table covers ceil(lengths[r] / page_size) pages with entries >= 0,
 *   and every slot page * page_size + page_size - 1 fits in int32;
 *   the lengths given to topk_select_paged equal those the plan was built from.
 *
 * Split rows
 * ----------
 * The page splits a long row across an 8-CTA thread-block cluster and reduces
 * the CTAs' histograms across the cluster (Figure 2 caption). gfx950 has no
 * clusters: the library splits a long row across G workgroups of one
 * persistent grid, which merge their histograms through global atomics and then
 * wait for one another at a bounded spin barrier in device memory. That wait
 * is only guaranteed to end if every workgroup of the selection grid is
 * resident on the device at the same time. The library sizes the grid to the
 * device's co-resident capacity for one 512-lane workgroup per compute unit
 * (topk_query_sizes) and puts every split row's chunks in the grid's first
 * round, so an otherwise idle device always satisfies this. Work that other
 * streams or processes run on the device at the same time can occupy compute
 * units and delay some of the grid's workgroups; the split rows' workgroups
 * that started then poll until cfg->spin_limit runs out, set
 * TOPK_DEVICE_SPIN_TIMEOUT in the workspace status word and exit (the kernel
 * always ends). Those rows' outputs are then incomplete and the workspace
 * must be cleared with topk_workspace_init before its next use. The caller
 * sees this only through topk_read_status; it never hangs the device.
 */
#ifndef SPARSE_TOPK_H
#define SPARSE_TOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. A plain int32 rather than an enum type, so that any value a
 * caller passes back (topk_status_string) is a valid value of the type. */
typedef int32_t topk_status;
enum {
  TOPK_OK = 0,
  TOPK_ERR_INVALID_ARG = -1,     /* a host-checkable argument is out of range or NULL */
  TOPK_ERR_BUFFER_TOO_SMALL = -2,/* plan or workspace smaller than topk_query_sizes says */
  TOPK_ERR_UNSUPPORTED = -3,     /* forced path cannot serve the configured rows */
  TOPK_ERR_HIP = -4,             /* a HIP runtime call or kernel launch failed */
  TOPK_ERR_DEVICE = -5           /* topk_read_status: the device recorded an error */
};

/* Path selection (tests and tuning). AUTO lets the planner choose per row. */
enum {
  TOPK_PATH_AUTO = 0,
  TOPK_PATH_REGISTER = 1,  /* one workgroup per row, row held in registers (len <= topk_register_capacity()) */
  TOPK_PATH_SINGLE = 2,    /* one workgroup per row, streamed */
  TOPK_PATH_MULTI = 3      /* every row longer than k split across workgroups */
};

/* Host struct, read through the pointer and never retained. */
typedef struct {
  int32_t k;              /* 1 .. 2048 */
  int32_t max_rows;       /* rows the plan and workspace are sized for (>= 1) */
  int64_t max_len;        /* largest valid length of any row (>= 0, < 2^31) */
  int32_t force_path;     /* TOPK_PATH_* */
  int32_t wg_per_row;     /* 0 = planner's choice; > 0 fixes the workgroups per split row */
  int32_t cand_capacity;  /* 0 = default; > 0 caps the per-row boundary-candidate buffer
                             (rows whose boundary bin holds more use a re-streaming path) */
  int32_t min_chunk;      /* 0 = default; > 0 smallest chunk (elements) the planner splits to */
  int32_t spin_limit;     /* bound on the split-row wait (see "Split rows" above):
                             0 = default (2^21 polls, about 1 s); > 0 = at most this many polls;
                             -1 = give up without polling (tests the time-out path); else invalid */
  int32_t reserved[3];    /* must be zero */
} topk_config;

/*
 * Host only. Sizes in bytes of the plan buffer (written by topk_plan) and the
 * workspace (used by topk_select_paged) for `cfg` on the current HIP device.
 * Status: OK, INVALID_ARG (bad cfg or NULL outputs), HIP (device query failed).
 * Passage: none; the pages define no buffers. This is the library's own sizing
 * of the plan and the cross-workgroup state that replace the page's cluster.
 */
topk_status topk_query_sizes(const topk_config* cfg, size_t* plan_bytes, size_t* workspace_bytes);

/*
 * Passage: none (the library's own state, see "Split rows").
 * Enqueue a fill kernel that zeroes `workspace`. Required once before the
 * first topk_select_paged on a workspace, and again after topk_read_status
 * reports TOPK_ERR_DEVICE. topk_select_paged leaves the workspace zeroed for
 * the next call, so no per-call clearing is needed (or recorded in a graph).
 */
topk_status topk_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * The planning step (page: TopK-V2, paragraph on the planning kernel): a
 * device kernel reads `lengths` (int32[num_rows], device) and writes the work
 * list into `plan`. Run it once per forward; the plan stays valid for any
 * number of topk_select_paged calls whose lengths are the same values.
 * Batches of at most TOPK_IN_KERNEL_PLAN_ROWS rows are planned inside the
 * selection kernel instead (from the same lengths, with the same result), so
 * for them this call checks its arguments and enqueues nothing.
 * 0 <= num_rows <= cfg->max_rows. No host synchronisation.
 */
#define TOPK_IN_KERNEL_PLAN_ROWS 512
topk_status topk_plan(const topk_config* cfg, const int32_t* lengths, int32_t num_rows,
                      void* plan, size_t plan_bytes, void* stream);

/*
 * The fused selection and page-table transform (page: TopK-V2, Figures 2-4).
 *   scores          float[num_rows][score_row_stride], row-major; row r's valid
 *                   prefix is lengths[r]. score_row_stride >= cfg->max_len.
 *   block_table     int32; row r's table starts at block_table + r * bt_row_stride
 *                   (bt_row_stride == 0: one table shared by all rows).
 *   page_size       tokens per KV page, >= 1.
 *   out_slots       int32[num_rows][out_row_stride], out_row_stride >= k.
 *   out_indices     int32[num_rows][out_row_stride] or NULL.
 *   plan            written by topk_plan for the same cfg and lengths; not read
 *                   (and may be NULL) when num_rows <= TOPK_IN_KERNEL_PLAN_ROWS.
 *   workspace       >= topk_query_sizes bytes, zeroed once by topk_workspace_init.
 * Status: OK, INVALID_ARG, BUFFER_TOO_SMALL, UNSUPPORTED, HIP. No host synchronisation.
 */
topk_status topk_select_paged(const topk_config* cfg, const void* plan,
                              const float* scores, int64_t score_row_stride,
                              const int32_t* lengths, int32_t num_rows,
                              const int32_t* block_table, int64_t bt_row_stride,
                              int32_t page_size,
                              int32_t* out_slots, int32_t* out_indices, int64_t out_row_stride,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Passage: TopK-V2 text and Figure 4 (the kernel latency the page measures).
 * topk_select_paged for measurement: identical arguments, results and errors,
 * plus two HIP events (hipEvent_t, created by the caller, timing enabled)
 * that record the selection kernel's own start and end, as a kernel trace
 * reports them, rather than the stream position before and after it.
 * Both events are required (INVALID_ARG otherwise).
 */
topk_status topk_select_paged_timed(const topk_config* cfg, const void* plan,
                                    const float* scores, int64_t score_row_stride,
                                    const int32_t* lengths, int32_t num_rows,
                                    const int32_t* block_table, int64_t bt_row_stride,
                                    int32_t page_size,
                                    int32_t* out_slots, int32_t* out_indices, int64_t out_row_stride,
                                    void* workspace, size_t workspace_bytes, void* stream,
                                    void* start_event, void* stop_event);

/*
 * Passage: none (the library's error reporting).
 * SYNCHRONISES `stream`. Copies the device status word of `workspace` into
 * *host_status (host pointer): 0, or a bitwise OR of TOPK_DEVICE_* flags.
 * Returns TOPK_ERR_DEVICE when the word is non-zero.
 */
enum {
  TOPK_DEVICE_SPIN_TIMEOUT = 1,  /* workgroups of a split row never all arrived */
  TOPK_DEVICE_PLAN_MISMATCH = 2, /* plan built for another k or never written */
  TOPK_DEVICE_BAD_LENGTH = 4,    /* a length outside [0, max_len] */
  TOPK_DEVICE_INTERNAL = 8       /* an internal consistency check failed */
};
topk_status topk_read_status(const void* workspace, size_t workspace_bytes,
                             int32_t* host_status, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * selection as topk_select_paged, with no plan buffer and no workspace
 * argument. The cross-workgroup state lives in a library-owned device array of
 * TOPK_NOALLOC_SCRATCH_BYTES per GPU (held until the process ends). The
 * call allocates nothing. It enqueues a fill kernel that clears the part of
 * that array the call uses, then the selection kernel.
 *   Arguments as for topk_select_paged. The batch must be planned inside the
 *   selection kernel: num_rows <= TOPK_IN_KERNEL_PLAN_ROWS, else UNSUPPORTED.
 *   The workspace topk_query_sizes reports for cfg must fit the array, else
 *   BUFFER_TOO_SMALL (nothing enqueued).
 *   device_status   int32 (device) or NULL: when given, the kernel ORs its
 *                   TOPK_DEVICE_* flags into it (the caller zeroes it first);
 *                   when NULL, they are not reported.
 * Every call on one GPU shares that GPU's array: calls that can overlap on one
 * GPU (two streams, two threads) race and give undefined results. Status: OK,
 * INVALID_ARG, BUFFER_TOO_SMALL, UNSUPPORTED, HIP. No host synchronisation.
 */
#define TOPK_NOALLOC_SCRATCH_BYTES (16u << 20)
topk_status topk_select_paged_noalloc(const topk_config* cfg, const float* scores, int64_t score_row_stride,
                                      const int32_t* lengths, int32_t num_rows, const int32_t* block_table,
                                      int64_t bt_row_stride, int32_t page_size, int32_t* out_slots,
                                      int32_t* out_indices, int64_t out_row_stride, int32_t* device_status,
                                      void* stream);

/* Elements one workgroup holds in registers (the register path's row limit).
 * Passage: TopK-V2 text, the register-resident path for short rows; the
 * limit itself is this library's tile size. */
int64_t topk_register_capacity(void);

/*
 * Test hook for the key transform of the page's Figure 3 caption (FP32 score
 * rounded to FP16, mapped to an unsigned key ordered like the score; the top
 * 10 key bits select one of 1,024 bins). For each x[i] (device, n >= 0) it
 * writes what the selection kernel itself computes:
 *   bin_out[i]   = histogram bin of x[i], 0..1023 (-0.0 shares +0.0's bin)
 *   key32_out[i] = order-preserving unsigned key of the FP32 value of x[i]
 *                  (-0.0 shares +0.0's key), used by the exact refinement
 * Either output pointer may be NULL. Enqueued on `stream`.
 */
topk_status topk_debug_keys(const float* x, int64_t n, uint32_t* bin_out, uint32_t* key32_out, void* stream);

/*
 * Test hook for the coarse histogram and threshold bin (page: TopK-V2,
 * Figure 3 caption: each score's FP16 key selects one of 1,024 bins by its
 * upper 10 bits and the bin's counter is incremented; Figure 2 caption: the
 * reduction locates the bin holding the k-th largest score). For each row r
 * of scores (device, float[num_rows][score_row_stride], valid prefix
 * lengths[r] (device), 0 <= lengths[r] <= score_row_stride) it writes, with
 * the selection kernel's own binning and threshold scan:
 *   hist_out[r * 1024 + b]   scores of the valid prefix in ordered bin b
 *                            (device, uint32[num_rows][1024]); bins 15 (-inf)
 *                            to 1008 (+inf) hold every non-NaN score; bins
 *                            0-14 and 1009-1023 hold only NaN codes, and the
 *                            kernel counts its padding of a tile past the
 *                            row's end there (it never scans them);
 *   threshold_out[r * 3 + 0..2] = { b*, scores in bins above b*, scores in b* }
 *                            (device, uint32[num_rows][3]): b* is the bin with
 *                            above(b*) < k <= above(b*) + hist[b*]; for rows of
 *                            at most k scores, { 0xFFFFFFFF, 0, 0 }.
 * 1 <= k <= 2048. One workgroup per row; enqueued on `stream`. Status: OK,
 * INVALID_ARG (bad k, num_rows < 0, NULL pointer with num_rows > 0), HIP.
 */
topk_status topk_debug_histogram(const float* scores, int64_t score_row_stride, const int32_t* lengths,
                                 int32_t num_rows, int32_t k, uint32_t* hist_out, uint32_t* threshold_out,
                                 void* stream);

/*
 * Passage: none; a measurement aid for the roofline of the streaming step
 * (TopK-V2 text: each score row is read once).
 * Measurement hook: the device's streaming-read ceiling for this access
 * pattern. Reads the whole 16-byte vectors of x[0, n) (device, n >= 0,
 * 16-byte aligned) once with the selection kernel's loads (512-lane
 * workgroups, one per compute unit, each lane keeping 16 vectors in flight)
 * and writes one partial sum per workgroup to out[0, topk_stream_read_groups())
 * (device), so the reads cannot be elided. Enqueued on `stream`. When both
 * start_event and stop_event (hipEvent_t) are given, they record the
 * kernel's own start and end, as in topk_select_paged_timed; else pass NULL.
 * Status: OK, INVALID_ARG (NULL pointer with n > 0, misaligned x, n < 0,
 * only one event), HIP.
 */
topk_status topk_debug_stream_read(const float* x, int64_t n, float* out, void* stream, void* start_event,
                                   void* stop_event);
/* Partial sums topk_debug_stream_read writes (its grid). Passage: none. */
int32_t topk_stream_read_groups(void);

/* Passage: none. A static string describing `s` ("unknown status" for values
 * outside topk_status); never NULL, owned by the library. */
const char* topk_status_string(topk_status s);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_TOPK_H */
