/*
 * rnn.h - C ABI of the MI355X (gfx950) LSTM/GRU layer engine (librnn.so).
 *
 * One recurrent layer (one direction, or both) per call. Three calls share a
 * caller-owned workspace, in the order forward -> backward-data ->
 * backward-weights, like the cuDNN training triple wrapped on the SystemDS
 * LibMatrixCuDNN page ("singleLayerUnidirectionalRNNForward", "lstmBackward":
 * forward training fills a reserve space that the backward-data and
 * backward-weights calls then read).
 *
 * The equations are those of the popnn pages:
 *   LSTM (Lstm.cpp, "basicLstmCellForwardPass", "backwardStepImpl"):
 *     z = x W_ih^T + b_ih + h W_hh^T + b_hh, i,f,o = sigmoid, g = tanh,
 *     c_t = f*c_{t-1} + i*g, h_t = o*tanh(c_t).
 *   GRU (Gru.cpp, "basicGruCellForwardPass", "backwardStepImpl"):
 *     r,u = sigmoid(x W_i^T + b_i + h W_h^T + b_h),
 *     basic:       c = tanh(x W_ic^T + b_ic + (r*h) W_hc^T + b_hc),
 *     reset_after: c = tanh(x W_ic^T + b_ic + r*(h W_hc^T + b_hc))
 *                  ("gruCellForwardPassCalcUnitsResetAfter"),
 *     h_t = u*h_{t-1} + (1-u)*c.
 *
 * Layouts (all row-major, element type given by desc->dtype):
 *   x, dx   [T][B][I], row (t,b) at x + (t*B+b)*ldx    (ldx >= I)
 *   y, dy   [T][B][H], row (t,b) at y + (t*B+b)*ldy    (ldy >= H)
 *   h0,hT,c0,cT,dh0,dc0,dhT,dcT  [B][H] dense
 *   W_ih [G*H][I], W_hh [G*H][H], b_ih/b_hh [G*H]; row block k (H rows)
 *   holds gate gate_order[k]. G = 4 (LSTM), 3 (GRU).
 *   dW_ih, dW_hh, db_ih, db_hh: same shapes and order as the weights.
 * Strides let a bidirectional layer write its two halves of one [T][B][2H]
 * output (pass y + H and ldy = 2H for the reverse half), as the strided
 * OUTPUT_STRIDE rows of the persistent kernel on the CUDA fragment page.
 *
 * Bidirectional layer (direction 2): one call runs both directions, their
 * persistent kernels sharing one launch (each on half of the chip) when the
 * plan divides that way. Every per-direction array is stacked [2][...],
 * direction 0 first: W_ih [2][G*H][I], W_hh [2][G*H][H], b_ih/b_hh [2][G*H],
 * h0,hT,c0,cT,dh0,dc0,dhT,dcT [2][B][H], dW_ih/dW_hh/db_ih/db_hh likewise;
 * y and dy hold direction 0 in columns [0, H) and direction 1 in [H, 2H)
 * (ldy >= 2H, 0 = 2H); dx receives the sum of both directions (added to
 * dx's contents when accumulate != 0), and so does datt. lengths and att
 * apply to both directions. The workspace is twice a single direction's.
 *
 * Pointers: every tensor pointer is a device pointer, 16-byte aligned.
 * NULL h0/c0/dhT/dcT mean zeros; NULL hT/cT/dh0/dc0 are not written;
 * NULL dx skips the input-gradient product. c0/cT/dc0/dcT are ignored for GRU.
 *
 * Errors: every call returns RNN_OK (0) or a negative rnn_status. Argument
 * errors are detected on the host before any device work is queued. Calls are
 * asynchronous on `stream` (a hipStream_t; NULL = default stream); a device
 * time-out of the cross-workgroup step handshake is reported through
 * rnn_last_device_status() after the stream has been synchronised.
 *
 * Ownership: the caller owns every buffer. The library allocates no device
 * memory. The workspace written by rnn_fwd must be passed unchanged to
 * rnn_bwd_data and then rnn_bwd_weights for the same descriptor and inputs.
 * Calls that share a workspace must not overlap in time.
 */
#ifndef RNN_H_
#define RNN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum rnn_mode { RNN_LSTM = 0, RNN_GRU = 1 };
enum rnn_dtype { RNN_F32 = 0, RNN_BF16 = 1 };

/* gate ids used in gate_order */
enum { RNN_GATE_I = 0, RNN_GATE_F = 1, RNN_GATE_G = 2, RNN_GATE_O = 3 }; /* LSTM */
enum { RNN_GATE_R = 0, RNN_GATE_U = 1, RNN_GATE_C = 2 };                 /* GRU  */

typedef enum rnn_status {
  RNN_OK = 0,
  RNN_ERR_INVALID_ARG = -1,         /* null required pointer, bad size, mode, dtype, order */
  RNN_ERR_WORKSPACE_TOO_SMALL = -2, /* ws_bytes < rnn_workspace_bytes(desc) */
  RNN_ERR_UNSUPPORTED = -3,         /* shape outside what the kernels handle (alignment,
                                       H or I granularity, persistent grid not co-resident) */
  RNN_ERR_DEVICE = -4,              /* a HIP runtime call failed */
  RNN_ERR_TIMEOUT = -5              /* (device status) step handshake timed out */
} rnn_status;

typedef struct rnn_desc {
  int mode;          /* RNN_LSTM or RNN_GRU */
  int direction;     /* 0: t = 0..T-1; 1: t = T-1..0 (outputs stay at their own t);
                        2: both (bidirectional layer, see above) */
  int reset_after;   /* GRU only: 0 basic, 1 reset applied after the recurrent product */
  int gate_order[4]; /* gate_order[k] = gate id stored in row block k; a permutation of
                        0..G-1 (LSTM i,f,g,o = 0..3; GRU r,u,c = 0..2). Common orders:
                        LSTM {0,1,2,3} (i,f,g,o) and {1,0,2,3} (f,i,g,o); GRU {0,1,2} */
  int dtype;         /* RNN_F32 or RNN_BF16 storage; arithmetic accumulates in fp32
                        (RNN_F32 products run on the bf16 matrix cores, each
                        operand split exactly into three bf16 pieces and the six
                        leading piece products summed: results at fp32 rounding
                        level) */
  int T, B, I, H;    /* T,B >= 1; I % 8 == 0; H % 16 == 0 */
  long long ldx;     /* row stride of x/dx in elements, 0 = I; multiple of 8 */
  long long ldy;     /* row stride of y/dy in elements, 0 = H (direction 2: 2H); multiple of 8 */
  const int* lengths; /* optional, device memory: int32 lengths[B], the number of
                        steps of each batch row (values clamped to [0, T]); NULL =
                        every row has T steps. Step t is active for row b iff
                        t < lengths[b] (popnn Gru.cpp / Lstm.cpp per-batch step
                        limits, "batchwiseFlags": masked gates, zero-filled output
                        sequence, latched state): an inactive step writes zero to
                        y and dx, keeps the state and passes the carried gradients
                        through, so hT/cT are the state after the row's last
                        active step and dh0/dc0 the gradients reaching its first;
                        in direction 1 a row starts at its own step lengths[b]-1
                        from h0/c0. The same array must be given to the three
                        calls and stay unchanged between them, and the y passed
                        to the backward calls is rnn_fwd's (zero past each
                        row's length). */
  const void* att;    /* optional, GRU only (else RNN_ERR_INVALID_ARG), device
                        memory of the storage type: AUGRU attention scores
                        att[T][B], row t*B+b (popnn Gru.cpp, the attention-score
                        forward and backward steps): the update gate u of step
                        t, row b is replaced by (1 - att[t][b]) * u in the state
                        update h = u*h_prev + (1-u)*c. NULL = plain GRU. The
                        same array must be given to the three calls. */
  int recompute;      /* LSTM only (else 0): 0 = rnn_fwd keeps the cell-state
                        sequence for the backward calls; 1 = it keeps only the
                        four gates and rnn_bwd_data rebuilds the cell states
                        from them and c0 before BPTT (popnn Lstm.cpp,
                        "cellAndTanh" recomputation): T*B*H fewer workspace
                        elements for one extra elementwise pass. */
  int dw_hh_mode;     /* 0 = the recurrent-weight gradient is accumulated inside
                        the BPTT kernel of rnn_bwd_data where its plan allows
                        (fp32, reset-after GRU or LSTM, batch groups of <= 8
                        rows; rnn_plan_t.fused_dw) and rnn_bwd_weights only
                        sums the per-group partials, the weight update folded
                        into the backward steps as the popnn LSTM/GRU pages'
                        backward-with-weight-update does; 1 = dW_hh always
                        from the separate product over the saved gate
                        gradients. Same value for both backward calls. */
  int stepwise;       /* 0 = the persistent kernels where a plan with a co-resident
                        grid fits the shape and device (rnn_plan_query), else one
                        recurrent product and one cell kernel per step (the
                        CUDA fragment page's per-step structure, and popnn's
                        step loop: the same equations, any H and B the
                        workspace holds, slower); 1 = the per-step path
                        always. */
} rnn_desc_t;

/* Bytes of workspace the three calls need for this descriptor (0 if the
 * descriptor is invalid). The workspace plays the role of the reserve space
 * that the SystemDS LibMatrixCuDNN page sizes through its RNN algorithm
 * object and hands to the forward-training, backward-data and
 * backward-weights calls ("lstm" / "lstmBackward"): it holds the saved
 * per-step activations, the gate gradients, step counters and scratch.
 * Pure host computation; needs no device. */
size_t rnn_workspace_bytes(const rnn_desc_t* desc);

/* Forward over the sequence (popnn Lstm.cpp "lstmFwd" / Gru.cpp "gruFwd",
 * one "basicLstmCellForwardPass" / "basicGruCellForwardPass" per step, the
 * input-weight product hoisted over all steps as "calcSequenceWeightedInputs"
 * does; the forward-training call of the SystemDS page's
 * "singleLayerUnidirectionalRNNForward"): y [T][B][H] (every step), hT and cT
 * [B][H] (the state after the last processed step), and the per-step
 * activations that the backward calls read, kept in the workspace.
 * Required: x, W_ih, W_hh, b_ih, b_hh, y; h0/c0 NULL = zero initial state
 * (the CUDA fragment page's `cx == NULL` test); hT/cT NULL = not written.
 * Returns RNN_ERR_INVALID_ARG for a bad descriptor, a NULL required pointer
 * or a pointer that is not 16-byte aligned, RNN_ERR_WORKSPACE_TOO_SMALL,
 * RNN_ERR_UNSUPPORTED for a shape the kernels do not handle, RNN_ERR_DEVICE
 * if a launch fails; nothing is queued when an error is returned.
 * Queues: the input projection GEMM, then one persistent recurrent kernel. */
int rnn_fwd(const rnn_desc_t* desc, const void* x, const void* h0, const void* c0,
            const void* W_ih, const void* W_hh, const void* b_ih, const void* b_hh,
            void* y, void* hT, void* cT, void* workspace, size_t ws_bytes, void* stream);

/* Forward over the sequence with no allocation and no workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): rnn_fwd,
 * same arguments, outputs and errors, with its workspace in a static device
 * array of RNN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends. A descriptor whose rnn_workspace_bytes()
 * exceeds that size is refused with RNN_ERR_WORKSPACE_TOO_SMALL before any
 * device work. The call allocates nothing (no hipMalloc, no library
 * allocation). All calls on one GPU share that GPU's array, which keeps the
 * last call's contents: calls that overlap in time on one GPU race, and the
 * saved activations it leaves are not meant for the backward calls (they
 * take a caller-owned workspace written by rnn_fwd). The first call on a
 * device looks up the array's device address (RNN_ERR_DEVICE if that
 * fails). */
#define RNN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int rnn_fwd_noalloc(const rnn_desc_t* desc, const void* x, const void* h0, const void* c0,
                    const void* W_ih, const void* W_hh, const void* b_ih, const void* b_hh,
                    void* y, void* hT, void* cT, void* stream);

/* Backward through time for the data gradients (popnn Lstm.cpp
 * "backwardStepImpl" and Gru.cpp "backwardStepImpl" /
 * "backwardStepImplResetAfter" per step, in reverse step order; the
 * persistent backward-data kernel of the CUDA fragment page; the
 * backward-data call of the SystemDS page's "lstmBackward"):
 * dx [T][B][I] (overwritten, or added to when accumulate != 0), dh0, dc0
 * [B][H], from dy at every step and the final-state gradients dhT/dcT.
 * With attention scores (desc->att), datt [T][B] (storage type; NULL = not
 * written) receives their gradient, minus the sum over hidden units of the
 * scaled update gate's gradient times the unscaled gate, zero past a row's
 * length; it follows the same overwrite / accumulate rule as dx.
 * Required: W_ih, W_hh, y, dy; y, h0 and c0 are the values given to /
 * produced by rnn_fwd with this workspace. dhT/dcT NULL = zero; dh0/dc0 NULL
 * = not written (the CUDA fragment page's `dhx != NULL`, `dcx != NULL`
 * tests); dx NULL skips the input-gradient product. The per-step gate
 * gradients are kept in the workspace for rnn_bwd_weights. Errors as for
 * rnn_fwd. Queues: one persistent reverse-time kernel, the score-gradient
 * sum (with datt), then the dx GEMM. */
int rnn_bwd_data(const rnn_desc_t* desc, const void* W_ih, const void* W_hh,
                 const void* h0, const void* c0, const void* y, const void* dy,
                 const void* dhT, const void* dcT, void* dx, void* dh0, void* dc0,
                 void* datt, int accumulate, void* workspace, size_t ws_bytes, void* stream);

/* Weight gradients summed over every (t, b) (popnn Lstm.cpp
 * "basicLstmParamUpdate", Gru.cpp "basicGruParamUpdate"; the
 * backward-weights call of the SystemDS page's "lstmBackward"):
 * dW_ih = sum dG^T x, dW_hh = sum dG_h^T h_{t-1} (h_{-1} = h0), db_ih,
 * db_hh, in the weights' shapes and gate order. accumulate != 0 adds to the
 * existing contents (popnn zeroes its accumulators and then adds), otherwise
 * they are overwritten. Any of the four outputs may be NULL to skip it.
 * Required: x, y (rnn_fwd's); the workspace written by rnn_fwd and then
 * rnn_bwd_data. Errors as for rnn_fwd. Queues: the dW GEMMs and the bias
 * reductions. */
int rnn_bwd_weights(const rnn_desc_t* desc, const void* x, const void* h0, const void* y,
                    void* dW_ih, void* dW_hh, void* db_ih, void* db_hh, int accumulate,
                    void* workspace, size_t ws_bytes, void* stream);

/* Device status word of the workspace (RNN_OK or RNN_ERR_TIMEOUT) after the
 * caller has synchronised the stream of the last call; the device-side
 * counterpart of the status checks that the SystemDS page's "checkStatus"
 * performs on every library call. Reads 4 bytes with a blocking copy;
 * RNN_ERR_INVALID_ARG for a NULL workspace, RNN_ERR_DEVICE if the copy
 * fails. */
int rnn_last_device_status(const void* workspace);

/* Static description of a status code (never NULL; "unknown status" for a
 * value that is not an rnn_status), as the SystemDS page's "checkStatus"
 * turns a library status into its message. */
const char* rnn_status_string(int status);

/* Time-out of the cross-workgroup step handshake for the calls queued after
 * this one, process-wide (the bounded waits of the persistent kernels;
 * default 10 s). The CUDA fragment page's persistent kernel spins on its
 * step data with no bound; here every wait is bounded and reports
 * RNN_ERR_TIMEOUT through rnn_last_device_status. 0 restores the default; a
 * negative value makes every wait give up at once, so a call completes with
 * RNN_ERR_TIMEOUT in its device status and undefined outputs (a way to
 * exercise the error path). Returns RNN_OK. */
int rnn_set_handshake_timeout(double seconds);

/* Plan of the persistent recurrent kernel of one pass (0 = forward,
 * 1 = backward through time) for this descriptor: how the batch rows and
 * hidden units are split over workgroups, which the CUDA fragment page's
 * persistent kernel fixes at compile time (its block and batch tiling) and
 * the popnn pages leave to the IPU planner. A persistent grid only runs when
 * all its workgroups are resident at once, since every workgroup waits for
 * the others at every step: when no instantiated kernel fits `cu_count`
 * compute units with `wg_per_cu` workgroups co-resident per CU (or the
 * descriptor sets `stepwise`), the layer takes the per-step path and the
 * result has stepwise = 1. cu_count = 0 queries the current device,
 * wg_per_cu = 0 asks the HIP runtime for the kernel's occupancy (both need
 * a GPU); with both given the call is pure host computation, the same
 * decision rnn_fwd / rnn_bwd_data / rnn_bwd_weights take before launching.
 * Returns RNN_OK with *out filled, RNN_ERR_INVALID_ARG (bad descriptor,
 * pass, counts or NULL out), RNN_ERR_UNSUPPORTED (shape outside the
 * granularity the kernels need), or RNN_ERR_DEVICE. */
typedef struct rnn_plan {
  int groups;       /* batch groups (each runs its own recurrence) */
  int rows;         /* batch rows per group */
  int slices;       /* hidden slices per group (workgroups of a group) */
  int units;        /* hidden units per slice */
  int waves;        /* 64-wide waves per workgroup */
  int workgroups;   /* working workgroups of the launch (both directions when dual) */
  int dual;         /* 1: the two directions of a bidirectional layer share one launch */
  int ring;         /* exchange of the step vector: 0 rows of y / dG, 1 tiled ring, 2 packed ring */
  int xcd_span;     /* XCDs one batch group covers */
  double model_us_per_step; /* the planner's modelled time per step */
  int blocks;       /* blocks launched: workgroups, or more when groups are padded to whole
                       XCDs (the extra blocks return at once) */
  int fused_dw;     /* pass 1: the BPTT kernel accumulates dW_hh itself (dw_hh_mode 0, a
                       plan with the fused variant, and the planner's model finding that
                       its extra per-step products cost less than the separate product) */
  int stepwise;     /* 1: no persistent grid (none fits, or the descriptor asks for the
                       per-step path); the other fields are then zero */
} rnn_plan_t;
int rnn_plan_query(const rnn_desc_t* desc, int pass, int cu_count, int wg_per_cu, rnn_plan_t* out);

/* Measurement probe of the step exchange (the per-step wait of the CUDA
 * fragment page's persistent kernel, here the step counters and exchange
 * ring): queues, for pass 0 (forward) or 1 (backward through time), a
 * persistent kernel on exactly the grid that rnn_fwd / rnn_bwd_data would
 * launch for this descriptor, which runs the T steps of the exchange alone:
 * the same placement check, counters, per-wave waits, exchange-ring loads and
 * stores, with no contraction and no gate arithmetic. Its time divided by T
 * is the floor that the exchange puts under a step. Takes a workspace as
 * rnn_fwd does (its status word and counters are overwritten; nothing else
 * the layer calls keep there is touched beyond the exchange ring). Returns
 * RNN_ERR_UNSUPPORTED for the basic GRU and plans without an exchange ring,
 * else as rnn_fwd. */
int rnn_handshake_probe(const rnn_desc_t* desc, int pass, void* workspace, size_t ws_bytes, void* stream);

/* Optional kernel timing, for measurement tools (the tracing hook of the
 * layer API; off by default). While enabled, every kernel the library queues
 * is bracketed by two HIP events recorded on the call's stream, under a label
 * naming the step of the layer it performs: "fill", "proj_gemm" (input
 * projection), "rec_fwd" (persistent forward), "rec_bwd" (persistent BPTT),
 * "dx_gemm", "dw_gemm", "db_colsum". Not thread-safe; enable it from one
 * thread around the calls to be timed. */
typedef struct rnn_kernel_time {
  char name[32];
  long long launches;
  double total_ms;
} rnn_kernel_time_t;

/* on != 0 starts recording, 0 stops. The library's HIP events are destroyed
 * once recording is off and every recorded pair has been read, so none is
 * alive at process exit. Returns RNN_OK. */
int rnn_profile_enable(int on);

/* Waits for every recorded event, folds the durations into per-label totals
 * and writes up to `max` entries to `out` (which may be NULL to only count).
 * reset != 0 clears the totals afterwards. Returns the number of labels, or
 * RNN_ERR_DEVICE if an event could not be read. */
int rnn_profile_read(rnn_kernel_time_t* out, int max, int reset);

#ifdef __cplusplus
}
#endif
#endif /* RNN_H_ */
