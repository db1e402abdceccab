/*
 * linrec.h -- C ABI of the MI355X (gfx950) linear-recurrence scan library.
 *
 * The operation is the channel-wise first-order linear recurrence
 *
 *     h[i,0,d] = b[i,0,d]
 *     h[i,t,d] = a[i,t,d] * h[i,t-1,d] + b[i,t,d]        t = 1 .. L-1
 *
 * for every batch row i < B and channel d < D, over (B, L, D) fp32 tensors with D
 * contiguous: the problem statement of the POPCORNBENCH "Kimi-K2.6 l1_p9" and
 * "FW-GLM-5-1 l1_p9" transcripts.  It is evaluated as an associative scan over
 * affine pairs: applying (a1, b1) and then (a2, b2) is the pair
 * (a2*a1, a2*b1 + b2), with identity (1, 0), and h is the second component of
 * the inclusive scan from a zero state (the operator derivation in the first
 * reasoning block of the Kimi-K2.6 l1_p9 transcript).  Only the running h has
 * to cross a chunk boundary (the running-carry passage of the same block).
 * The result is any valid bracketing of that scan in fp32 with fused
 * multiply-add, so it is not bitwise unique; it matches a float64 sequential
 * evaluation within 1e-4 * (1 + |h|) per element on the tested workloads.
 * linrec_scan_ex adds strided operands, bf16/fp16 storage, an initial and a
 * final state, and the reverse-time form.
 *
 * All entry points are host functions; apart from linrec_device_timeouts and
 * linrec_release, none of them synchronises the device.
 * No C++ or PyTorch types appear in this interface.
 */
#ifndef LINREC_H
#define LINREC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum linrec_status {
    LINREC_OK = 0,                  /* done, or enqueued on the stream                        */
    LINREC_ERR_INVALID_ARGUMENT = 1,/* negative size, size overflow, null or non-device buffer,
                                       buffer too small for B*L*D floats, or device mismatch   */
    LINREC_ERR_OVERLAP = 2,         /* an output buffer overlaps another buffer               */
    LINREC_ERR_HIP = 3,             /* a HIP runtime call or the kernel launch failed         */
    LINREC_ERR_OUT_OF_MEMORY = 4    /* the internal workspace could not be allocated          */
} linrec_status;

/*
 * linrec_scan -- h = scan of the recurrence above over every (i, d) channel.
 *
 *   a, b   input device buffers, B*L*D fp32 each, layout (B, L, D) row-major:
 *          element (i, t, d) at index (i*L + t)*D + d.  a[i,0,d] is never
 *          used: the state before t = 0 is zero, so h[i,0,d] = b[i,0,d].
 *   h      output device buffer, B*L*D fp32, same layout.  Must not overlap a
 *          or b (a and b may alias each other).
 *   B,L,D  sizes, each >= 0.  Any of them 0 is a successful no-op.
 *   stream hipStream_t to enqueue on, or NULL for the null stream.
 *
 * Ownership: the three buffers belong to the caller and must stay valid until
 * the work on `stream` completes; the library never frees them.  They must be
 * device memory of the current HIP device, each inside one allocation of at
 * least B*L*D*4 bytes (checked with the HIP runtime before launch).
 *
 * Workspace: when L spans several tiles and the tiles must look back across
 * workgroups, the call uses a workspace of status words.  The library keeps
 * one per (device, stream): it allocates it on the first call on that stream
 * that needs one (hipMalloc, then a clear enqueued on that stream before the
 * scan), replaces it with a larger one when a shape needs more, and frees all
 * of them in linrec_release().  A replaced workspace is kept, not freed, until then (a
 * graph captured with it may still be replayed).  Calls on one stream are
 * ordered, and calls on different streams use different workspaces, so
 * concurrent streams never share status words.  Each stream that makes such
 * calls holds its own workspace (a few MB for shapes like B=2 L=262144 D=64)
 * until linrec_release().  linrec_scan_ws takes the workspace from the caller
 * instead.  When the persistent workgroups can take whole (batch row, channel
 * slab) sequences, 1 to 4 each, the carry stays inside each workgroup and the
 * call touches no workspace.
 *
 * Graph capture: a call enqueues kernel launches only (no memset, no copy), so
 * it can be captured into a HIP graph and replayed, provided the workspace it
 * needs already exists: make one call of the same or a larger shape on the
 * capturing stream before capturing (a call that would have to allocate while
 * its stream is captured returns LINREC_ERR_INVALID_ARGUMENT), or pass a
 * workspace to linrec_scan_ws.  Replays need no host work between them: each
 * call's lookback epoch advances inside the kernel.  A captured call keeps
 * using the workspace it was captured with, so a replay must be ordered with
 * the other calls that use that workspace (those on the stream it was
 * captured on).
 *
 * Alignment: buffers must be aligned to 4 bytes (any fp32 array is): 16-byte
 * aligned buffers with D % 4 == 0 use 128-bit accesses, anything else the
 * 32-bit form of the same kernel.
 *
 * Errors: returns a status and never aborts; the message for the calling
 * thread's last failure is linrec_last_error_message().  LINREC_OK means the
 * work is enqueued; a device fault would surface at the caller's next
 * synchronisation.
 *
 * Environment: LINREC_TILE="t=<steps per lane>,w=<data waves per workgroup>,
 * vec=<1|4>,p=<lanes per row>,q=<workgroups per CU>,m=<0|1|2>,l=<0|1>,x=<0|1>"
 * overrides the tile shape, the kernel (m=0: persistent workgroups that take
 * tiles in turn; m=1: one workgroup per tile; m=2: as m=0, except that where
 * the carry stays local the relay kernel runs it, whose carry wave also does
 * the scan across the lanes of each tile, one tile behind the data waves;
 * with w > 2 or slabs wider than 64 channels, m=2 plans as m=0), whether
 * persistent workgroups
 * may keep the carry local (l=1, the default; l=0 makes every tile look back),
 * whether channel slabs narrower than a 128-byte line are grouped so that the
 * slabs sharing a line run on one XCD (x=1, the default; x=0 keeps dispatch
 * order) and the launch size the library picks (each key optional; unsupported
 * values are rejected with LINREC_ERR_INVALID_ARGUMENT).
 * LINREC_SPIN_LIMIT=<n> overrides how many times a tile polls a predecessor's
 * status before it recomputes that predecessor's pair from a and b itself
 * (see linrec_device_timeouts); results are the same either way, so it exists
 * to exercise that path and is not a tuning knob.
 */
linrec_status linrec_scan(const float *a, const float *b, float *h,
                          int64_t B, int64_t L, int64_t D, void *stream);

/*
 * linrec_plan -- how linrec_scan would run a shape: the tile it picks (after
 * any LINREC_TILE override), the launch size and the workspace it needs.
 */
typedef struct linrec_plan {
    int32_t vec;             /* channels per lane: 4 (128-bit accesses) or 1           */
    int32_t steps_per_lane;  /* consecutive time steps each lane keeps in registers    */
    int32_t waves;           /* 64-lane data wavefronts per workgroup (plus carry ones) */
    int32_t lanes_per_row;   /* lanes that share one time step of a channel slab       */
    int64_t steps_per_tile;  /* time steps one workgroup covers                        */
    int64_t chunks;          /* tiles along L for one (batch row, channel slab)        */
    int64_t tiles;           /* tiles of the problem (0 if empty); mode 1 launches one
                                workgroup per tile, modes 0 and 2 at most as many as
                                fit                                                    */
    size_t workspace_bytes;  /* device workspace the tiles need if they look back (0
                                when chunks <= 1); unused when the carry stays local  */
    int32_t mode;            /* 0: persistent workgroups take tiles in turn;
                                1: one workgroup per tile;
                                2: as 0, with the relay kernel where the carry stays
                                local (one carry wave scans each tile's lanes, one
                                tile behind the data waves)                            */
} linrec_plan;

/*
 * linrec_scan_plan -- fills *plan for a linrec_scan of shape (B, L, D) whose
 * buffers are 16-byte aligned (aligned16 != 0) or not, on a 256-CU MI355X.
 * Pure host arithmetic, no HIP call.  Returns LINREC_ERR_INVALID_ARGUMENT for negative sizes,
 * B*L*D*8 beyond 2^63 - 1 (every entry point applies this limit), more than 2^31 - 1 tiles,
 * an unsupported LINREC_TILE or a null plan.
 */
linrec_status linrec_scan_plan(int64_t B, int64_t L, int64_t D, int aligned16, linrec_plan *plan);

/* Storage type of a, b and h in linrec_scan_ex (arithmetic is always fp32). */
typedef enum linrec_dtype {
    LINREC_F32 = 0,   /* IEEE binary32                                                  */
    LINREC_BF16 = 1,  /* bfloat16: widened exactly on load, rounded to nearest even on store */
    LINREC_F16 = 2    /* IEEE binary16: same; values beyond its range become infinite    */
} linrec_dtype;

/* One (B, L, D) operand: element (i, t, d) at ptr[i*stride_b + t*stride_l + d],
 * strides in elements of the operand's storage type, each >= 0 (0 repeats a
 * row: e.g. one decay a shared by every batch row). */
typedef struct linrec_operand {
    const void *ptr;
    int64_t stride_b;
    int64_t stride_l;
} linrec_operand;

/*
 * linrec_scan_desc -- a generalised linrec_scan.
 *
 *   B, L, D   sizes, each >= 0.
 *   dtype     linrec_dtype of a, b and h.
 *   reverse   0: the recurrence runs forward in t, as in linrec_scan.
 *             1: it runs backward: h[i,L-1,d] = b[i,L-1,d] and
 *                h[i,t,d] = a[i,t,d] * h[i,t+1,d] + b[i,t,d] for t = L-2 .. 0
 *                (the time reversal of the recurrence).
 *             2: it runs backward with each decay taken one time step ahead:
 *                h[i,L-1,d] = b[i,L-1,d] (plus h_init[i,d], with decay 1) and
 *                h[i,t,d] = a[i,t+1,d] * h[i,t+1,d] + b[i,t,d].  Over an
 *                incoming gradient g as b, this is dLoss/db of the forward
 *                scan over the same a, read without a shifted copy of a;
 *                dLoss/da[t] is then dLoss/db[t] * h[t-1] of the forward scan.
 *                A sequence taken in pieces chains through
 *                h_init = a[:, L] * (the next piece's result at its first
 *                step).  a[i,0,d] is never read.
 *             The backward forms are not on the pages that define the forward
 *             recurrence.
 *   a, b, h   operands; h.ptr is written (cast away its const).  h's rows
 *             (i, t) must not overlap one another, checked as nesting: taking
 *             h's batch and time dimensions in increasing stride, each stride
 *             (of a dimension longer than 1) is at least the elements that one
 *             row and the smaller dimension span.  Contiguous, padded and
 *             transposed layouts nest; a layout whose time rows interleave
 *             with its batch rows is refused even where no two rows share an
 *             element.  h must not overlap a or b (a and b may overlap each
 *             other).
 *   h_init    NULL, or a (B, D) row-major fp32 device buffer: the state before
 *             the first step of the scan order, so that the first step is
 *             h = a * h_init + b instead of h = b (forward: t = 0; reverse:
 *             t = L-1; with reverse = 2 the decay of that step is 1).  This generalises the running carry between chunks
 *             of the pages' kernels (the running-carry passage of the first
 *             reasoning block of the Kimi-K2.6 l1_p9 transcript) to a carry
 *             between calls.
 *   h_final   NULL, or a (B, D) row-major fp32 device buffer that receives
 *             the state after the last step (forward: h[:, L-1, :]; reverse:
 *             h[:, 0, :]) before rounding to dtype; with L == 0 it receives
 *             h_init (or zeros).  Scanning a long sequence in pieces, each
 *             piece's h_final passed as the next one's h_init, gives the same
 *             result as one call within rounding.  Must not overlap any other
 *             buffer; h_init must not overlap h.
 *
 * 128-bit (fp32) or 64-bit (16-bit) accesses are used when D % 4 == 0, every
 * stride is a multiple of 4 and a, b, h are aligned to 4 elements; anything
 * else takes the one-channel-per-lane form of the same kernels.
 */
typedef struct linrec_scan_desc {
    int64_t B, L, D;
    int32_t dtype;
    int32_t reverse;
    linrec_operand a, b, h;
    const float *h_init;
    float *h_final;
} linrec_scan_desc;

/*
 * linrec_scan_ex -- the scan described by *desc, enqueued on `stream`.
 * Ownership, workspace, errors and environment as for linrec_scan; every
 * buffer is checked to lie inside one device allocation of the current
 * device that holds the elements the strides reach.  Returns
 * LINREC_ERR_INVALID_ARGUMENT for a null desc, bad sizes, strides or dtype,
 * rows of h that overlap one another, a, b or h not aligned to its element
 * size, h_init or h_final not aligned to 4 bytes, a tile of an operand that
 * would span 1 GiB or more (huge time strides), or bad buffers;
 * LINREC_ERR_OVERLAP when a written buffer overlaps another one.
 */
linrec_status linrec_scan_ex(const linrec_scan_desc *desc, void *stream);

/* linrec_scan_ex_plan -- fills *plan for linrec_scan_ex(desc) (pure host
 * arithmetic on the sizes, strides, dtype and pointer alignment; no HIP call,
 * buffers are not checked). */
linrec_status linrec_scan_ex_plan(const linrec_scan_desc *desc, linrec_plan *plan);

/*
 * Caller-provided workspaces -- for callers that run scans concurrently on
 * several streams of one device and want to manage the memory themselves, or
 * that capture graphs without a warm-up call.  Same operation, arguments,
 * ownership, errors and environment as linrec_scan / linrec_scan_ex, except
 * that the lookback workspace (see "Workspace" above) is the caller's:
 *
 *   workspace        device memory of the current device, 256-byte aligned,
 *                    at least the bytes the *_workspace_bytes functions give,
 *                    overlapping no operand, and ZERO-FILLED before its first
 *                    use, the clear ordered before that call (e.g.
 *                    hipMemsetAsync on the call's stream, or a hipMemset
 *                    followed by hipDeviceSynchronize: a plain hipMemset runs
 *                    on the null stream, which non-blocking streams do not
 *                    wait for).  The library keeps it consistent
 *                    from call to call afterwards (every 2^29 calls on one
 *                    workspace, a call also enqueues a clear of it on its
 *                    stream).  It may serve calls of any shape.
 *   workspace_bytes  its size.  May be anything (workspace may be NULL) when
 *                    the call needs no workspace.
 *
 * Calls that share one workspace must be ordered (one stream, or events);
 * calls with different workspaces may run concurrently.  These entry points
 * never allocate.  LINREC_ERR_INVALID_ARGUMENT when a needed workspace is
 * missing, too small, misaligned or not device memory of the current device;
 * LINREC_ERR_OVERLAP when it overlaps an operand.
 */
linrec_status linrec_scan_ws(const float *a, const float *b, float *h, int64_t B, int64_t L, int64_t D,
                             void *workspace, size_t workspace_bytes, void *stream);
linrec_status linrec_scan_ex_ws(const linrec_scan_desc *desc, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * linrec_scan_ex_noalloc -- linrec_scan_ex for callers that cannot allocate
 * device memory at all: code under HIP graph capture (including the first
 * call on a stream), tight serving loops, and harnesses that forbid
 * hipMalloc.  It runs the same kernels as linrec_scan_ex with the same
 * arguments, results, errors and environment, and calls no hipMalloc, hipFree
 * or other allocating routine.
 *
 * Its lookback workspace is a static 16 MiB array in the library's device
 * code, one per device, held from module load to process end.  A call whose
 * plan needs more (linrec_scan_ex_workspace_bytes above 16 MiB, e.g. very
 * long chains of small tiles) returns LINREC_ERR_INVALID_ARGUMENT and
 * enqueues nothing; linrec_scan_ex_ws serves those.  Calls whose plan needs
 * no workspace (a local carry, a single chunk) do not touch it.
 *
 * Every call on a device shares that device's array, and each call leaves it
 * in the state the next one expects.  Calls that may overlap in time on one
 * device (different streams, or graph replays concurrent with other calls)
 * therefore race: order them on one stream.  The first call on a device
 * enqueues a clear of the array (a fill kernel, no memset) on its stream
 * before the scan.  If that call is being captured, the clear is recorded in
 * the graph, so each replay clears the array first, and the next eager call
 * clears it again.
 */
linrec_status linrec_scan_ex_noalloc(const linrec_scan_desc *desc, void *stream);

/* Workspace bytes a linrec_scan_ws call of shape (B, L, D) may need on the
 * current device, whatever the buffers' alignment (0: none, or invalid
 * sizes).  Host arithmetic plus a query of the device's CU count. */
size_t linrec_scan_workspace_bytes(int64_t B, int64_t L, int64_t D);

/* Workspace bytes linrec_scan_ex_ws(desc) may need on the current device, into
 * *bytes (0: none).  LINREC_ERR_INVALID_ARGUMENT for a null bytes or an
 * invalid desc (the checks of linrec_scan_ex_plan). */
linrec_status linrec_scan_ex_workspace_bytes(const linrec_scan_desc *desc, size_t *bytes);

/* Static English text for a status code; "unknown status" for other values. */
const char *linrec_status_string(int status);

/* Message of the calling thread's most recent failure ("" if none).  The
 * pointer stays valid until that thread's next call into the library. */
const char *linrec_last_error_message(void);

/*
 * linrec_device_timeouts -- on the current device, summed over the library's
 * own workspaces since each was allocated (caller-provided workspaces keep
 * their own count): how many lookback wavefronts (at most four per workgroup
 * per call) stopped waiting for a predecessor's published carry at least once
 * and recomputed that predecessor's pair from the inputs instead.  The output is
 * correct either way; the count shows how often the cross-workgroup wait ran
 * out (normally 0).  Synchronises the device before reading.  Returns
 * LINREC_OK and stores the count in *count (0 when no workspace exists).
 */
linrec_status linrec_device_timeouts(uint64_t *count);

/* Frees the library's workspaces (those of every stream, and the ones larger
 * shapes replaced), synchronising each device that holds one first.  No other
 * thread may call into the library meanwhile.  A HIP graph that captured a
 * call whose tiles look back through a library workspace refers to freed
 * memory afterwards: do not replay it (capture it again after a first call
 * has allocated a new workspace).  The next call that needs a workspace
 * allocates a new one.  Caller-provided workspaces are not touched. */
void linrec_release(void);

#ifdef __cplusplus
}
#endif

#endif /* LINREC_H */
