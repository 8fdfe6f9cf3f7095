/*
 * tree_attn.h -- C ABI of libtreeattn.so: shared-prompt tree attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Method: "Splitting Prompt Prefill from Response Replay for Context-Parallel
 * Long-Context LLM Post-Training" (the AugTree paper).  A replay tree is one
 * shared prompt P and G response branches R_1..R_G (section 3.1).  The prompt
 * is prefilled once with causal attention and its K/V kept (section 3.2,
 * "Shared prompt prefill pass"); every response token then attends to the
 * whole prompt and to its own branch prefix, never to a sibling (section 3.2,
 * Eq. 1).  Prompt K/V gradients are the sum over all branches (section 3.2,
 * Eq. 2) and flow back through the prefill (section 3.2, "Exact many-to-one
 * backward").  Attention per head is O = softmax(Q K^T * scale + M) V
 * (section 2.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Tensors are packed token-major and contiguous:
 *   prompt   Q/O/dQ/dO [sum_g P_g, Hq, d],   K/V/dK/dV [sum_g P_g, Hkv, d]
 *   response Q/O/dQ/dO [sum_i r_i,  Hq, d],  K/V/dK/dV [sum_i r_i,  Hkv, d]
 *   LSE [Hq, tokens] float32: natural log of sum_j exp(scale * q . k_j)
 *   over the visible keys of that row.
 * Branches of one group are consecutive in the response tensors.  Query
 * head h reads kv head floor(h * Hkv / Hq).  The causal masks include the
 * diagonal.
 * dtype.  TREE_ATTN_BF16 or TREE_ATTN_F32 for every I/O tensor; LSE, prompt
 * gradient seeds and merge partials are always float32.  Matrix products
 * accumulate in float32.
 * Memory.  Every tensor pointer is caller-owned device memory with a
 * 16-byte aligned base.  The library allocates no device memory (apart from
 * the static scratch array of tree_attn_replay_fwd_noalloc, which comes with
 * the code object on each GPU).  Scratch space comes from the caller through
 * (ws, ws_bytes), sized by
 * tree_attn_workspace_size(); its contents need not be preserved between
 * calls.  Host arrays (*_h) are read during the call only; device arrays
 * (*_d) and every tensor must stay valid until the enqueued work finishes.
 * The *_h and *_d copies of an offset array must hold the same values.
 * Streams.  Each call only enqueues work on `stream` (a hipStream_t; NULL is
 * the default stream) and never synchronises.  Calls that share workspace
 * must be ordered on one stream.
 * Sizes.  Token totals times Hq, and padded token totals (each prompt and
 * branch rounded up to 64) times the packed head count, must fit in int32;
 * head_dim * padded tokens * packed heads * element size must stay below
 * 4 GiB.  The packed head count is the largest power of two (at most 16)
 * dividing Hq / Hkv.  Larger problems are rejected with
 * TREE_ATTN_ERR_INVALID.
 * Determinism.  With the default dQ strategies no output is accumulated
 * with atomics: every partial sum is added in a fixed order, so repeated
 * calls give bit-identical results.  TREE_ATTN_DQ_FUSED (below) adds dQ
 * with float32 atomics; there dQ varies from call to call by rounding and
 * every other output stays bit-identical.
 * Errors.  0 on success, else a negative tree_attn_status.  Arguments are
 * checked on the host before any HIP call, so a rejected call enqueues
 * nothing and writes nothing.  TREE_ATTN_ERR_HIP reports a failed launch.
 * The library holds no global mutable state apart from the per-thread
 * timing hook below and the per-GPU static scratch of
 * tree_attn_replay_fwd_noalloc, and may be called from several host threads.
 */
#ifndef TREE_ATTN_H_
#define TREE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* tree_attn_stream_t; /* a hipStream_t */

typedef enum {
  TREE_ATTN_F32 = 0,
  TREE_ATTN_BF16 = 1
} tree_attn_dtype;

typedef enum {
  TREE_ATTN_OK = 0,
  TREE_ATTN_ERR_INVALID = -1,     /* null pointer, bad offsets, bad shape */
  TREE_ATTN_ERR_UNSUPPORTED = -2, /* dtype or head_dim not supported */
  TREE_ATTN_ERR_WORKSPACE = -3,   /* ws_bytes below the required size */
  TREE_ATTN_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
  TREE_ATTN_ERR_SCRATCH = -5      /* tree_attn_replay_fwd_noalloc: the problem needs more
                                     than TREE_ATTN_STATIC_SCRATCH_BYTES of scratch */
} tree_attn_status;

/*
 * How the two backward calls form dQ (the attention definition of section
 * 2.2 differentiated; S = scale Q K^T, P = softmax, dS = P (dP - D)):
 *   TREE_ATTN_DQ_SEPARATE  a query-stationary pass recomputes S and dP and
 *       forms dQ = scale dS K with no atomics (seven matrix products per
 *       tile, bit-deterministic);
 *   TREE_ATTN_DQ_FUSED     the key-stationary dK/dV kernel also forms dQ from
 *       the dS it holds (five products) and adds it into a float32
 *       accumulator with atomics; bf16 with head_dim 128 only (else
 *       TREE_ATTN_ERR_UNSUPPORTED), dQ not bit-deterministic;
 *   TREE_ATTN_DQ_AUTO      the library picks one per call from a cost model
 *       (section 3.4, "Cost model", in spirit).
 */
typedef enum {
  TREE_ATTN_DQ_AUTO = 0,
  TREE_ATTN_DQ_SEPARATE = 1,
  TREE_ATTN_DQ_FUSED = 2
} tree_attn_dq_strategy;

typedef enum {
  TREE_ATTN_OP_PREFILL = 0,
  TREE_ATTN_OP_REPLAY_FWD = 1,
  TREE_ATTN_OP_REPLAY_BWD = 2,
  TREE_ATTN_OP_PREFILL_BWD = 3
} tree_attn_op;

/*
 * A batch of replay trees T = (P, {R_i}) (section 3.1).
 * num_groups    n_g >= 1 prompts.
 * num_branches  total branches over all groups (>= 0).
 * num_q_heads, num_kv_heads  Hq, Hkv >= 1 with Hq % Hkv == 0.
 * head_dim      64 or 128.
 * dtype         a tree_attn_dtype.
 * softmax_scale the score scale; 1/sqrt(head_dim) is the paper's choice.
 * prompt_cu     [n_g + 1] non-decreasing token offsets of each prompt in the
 *               prompt tensors, prompt_cu[0] == 0 (P_g >= 0).
 * group_branch_cu [n_g + 1] non-decreasing, group g owns branches
 *               group_branch_cu[g] .. group_branch_cu[g+1]-1;
 *               group_branch_cu[0] == 0, group_branch_cu[n_g] == num_branches.
 * resp_cu       [num_branches + 1] non-decreasing token offsets of each
 *               branch in the response tensors, resp_cu[0] == 0 (r_i >= 0).
 * Each offset array is given twice: *_h in host memory, *_d in device
 * memory, with equal contents.  The device copies may be NULL only for an
 * entry point that does not read them (none of the four attention calls).
 * dq_strategy   a tree_attn_dq_strategy (0, the automatic choice, when the
 *               struct is zero-initialised); the workspace size depends on
 *               it, so size and call with the same value.
 * prompt_col_splits  0: the library's makespan model picks, for each of the
 *               replay query launches (forward, and dQ of the separate
 *               strategy), how many chunks it cuts each prompt column into
 *               (section 3.3: the chunks' partial states are merged); 1..64:
 *               that many chunks for both (1 = not split), for measurements
 *               and calibration.  The workspace size depends on it.
 * prompt_tile_split_rows  0: the library's rule picks how the replay
 *               backward splits a group's prompt key tiles over ranges of its
 *               branches (each range a work item writing float32 partial
 *               seeds, added in a fixed order); r > 0: each range reads at
 *               most r response rows (whole branches, at least one each;
 *               a value at or above a group's rows leaves it unsplit), for
 *               measurements and calibration.  The workspace size depends
 *               on it.
 */
typedef struct {
  int32_t num_groups;
  int32_t num_branches;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  float softmax_scale;
  const int32_t* prompt_cu_h;
  const int32_t* prompt_cu_d;
  const int32_t* group_branch_cu_h;
  const int32_t* group_branch_cu_d;
  const int32_t* resp_cu_h;
  const int32_t* resp_cu_d;
  int32_t dq_strategy;
  int32_t prompt_col_splits;
  int32_t prompt_tile_split_rows;
} tree_attn_problem;

/*
 * Bytes of workspace that entry point `op` (a tree_attn_op) needs for this
 * problem.  Writes *bytes; no HIP call.
 */
int tree_attn_workspace_size(const tree_attn_problem* problem, int op, size_t* bytes);

/*
 * Prompt prefill (section 3.2, "Shared prompt prefill pass"): causal
 * attention of each group's prompt over its own prompt, computed once per
 * group.
 *   in : q_p [sum P, Hq, d], k_p, v_p [sum P, Hkv, d]
 *   out: o_p [sum P, Hq, d], lse_p [Hq, sum P] (float32)
 * The caller keeps k_p / v_p as the prompt K/V state for replay.
 */
int tree_attn_prefill(const tree_attn_problem* problem, const void* q_p, const void* k_p,
                      const void* v_p, void* o_p, float* lse_p, void* ws, size_t ws_bytes,
                      tree_attn_stream_t stream);

/*
 * Response replay forward (section 3.2, "Response replay"; Eq. 1): row t of
 * branch i attends to every key of its group's prompt (no mask) and to keys
 * 0..t of branch i (causal).  Both parts share one online-softmax state per
 * row, which is the partial-state merge of section 3.3 done in registers.
 *   in : k_p, v_p [sum P, Hkv, d] (prompt K/V state from prefill),
 *        q_r [sum r, Hq, d], k_r, v_r [sum r, Hkv, d]
 *   out: o_r [sum r, Hq, d], lse_r [Hq, sum r] (float32)
 * With few response rows behind a long prompt, the prompt keys are cut into
 * chunks processed in parallel; their float32 partial states go through
 * the same merge as lse_merge() below.  The workspace size covers them.
 */
int tree_attn_replay_fwd(const tree_attn_problem* problem, const void* k_p, const void* v_p,
                         const void* q_r, const void* k_r, const void* v_r, void* o_r,
                         float* lse_r, void* ws, size_t ws_bytes, tree_attn_stream_t stream);

/*
 * Size of the library's static scratch array (one per GPU), used only by
 * tree_attn_replay_fwd_noalloc: 128 MiB.
 */
#define TREE_ATTN_STATIC_SCRATCH_BYTES (128u << 20)

/*
 * tree_attn_replay_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Arguments, layout and results are those
 * of tree_attn_replay_fwd (same kernels, bit-identical outputs); the caller
 * still provides every input and output tensor.
 * Scratch.  The work lists, transposed V copies and (for long prompts)
 * prompt-column partials go to a static device array of
 * TREE_ATTN_STATIC_SCRATCH_BYTES, one per GPU, allocated with the library's
 * code object on that GPU and held until the process ends.  The call itself
 * allocates nothing and frees nothing.  A problem whose scratch would not fit
 * (tree_attn_workspace_size(problem, TREE_ATTN_OP_REPLAY_FWD, ...) reports the
 * same size) returns TREE_ATTN_ERR_SCRATCH before any HIP call.
 * Sharing.  Every call on one GPU uses that GPU's array, and nothing in it
 * is kept from one call to the next.  Calls whose work overlaps on one GPU
 * (different streams or host threads without ordering) race on the array
 * and give undefined results: order them on one stream or synchronise.
 * Device.  `stream` must belong to the calling thread's current device
 * (else TREE_ATTN_ERR_INVALID).  The array's device address is looked up
 * once per device, on the first call made on it.
 */
int tree_attn_replay_fwd_noalloc(const tree_attn_problem* problem, const void* k_p,
                                 const void* v_p, const void* q_r, const void* k_r,
                                 const void* v_r, void* o_r, float* lse_r,
                                 tree_attn_stream_t stream);

/*
 * Response replay backward (section 3.2, Eq. 2).  Given the replay forward's
 * o_r, lse_r and the upstream gradient do_r:
 *   out: dq_r [sum r, Hq, d], dk_r, dv_r [sum r, Hkv, d] (I/O dtype), and
 *        dk_p_seed, dv_p_seed [sum P, Hkv, d] float32: the response rows'
 *        gradient on the prompt K/V, summed over every branch of the group
 *        and over the query heads of each kv head.  The seeds are
 *        overwritten, not accumulated.  Passing NULL for both skips them
 *        (a detached prompt); passing exactly one NULL is invalid.
 */
int tree_attn_replay_bwd(const tree_attn_problem* problem, const void* k_p, const void* v_p,
                         const void* q_r, const void* k_r, const void* v_r, const void* o_r,
                         const float* lse_r, const void* do_r, void* dq_r, void* dk_r,
                         void* dv_r, float* dk_p_seed, float* dv_p_seed, void* ws,
                         size_t ws_bytes, tree_attn_stream_t stream);

/*
 * Prompt prefill backward (section 3.2: prompt-state gradient seeds are
 * propagated through the original prefill).  Causal backward of the prompt
 * over itself, plus the seeds:
 *   dk_p = prefill term + dk_p_seed,  dv_p = prefill term + dv_p_seed,
 *   dq_p = prefill term.
 *   in : q_p, k_p, v_p, o_p, lse_p (from tree_attn_prefill), do_p,
 *        dk_p_seed, dv_p_seed float32 (from tree_attn_replay_bwd; both NULL
 *        means zero seeds; exactly one NULL is invalid)
 *   out: dq_p [sum P, Hq, d], dk_p, dv_p [sum P, Hkv, d] (I/O dtype)
 */
int tree_attn_prefill_bwd(const tree_attn_problem* problem, const void* q_p, const void* k_p,
                          const void* v_p, const void* o_p, const float* lse_p,
                          const void* do_p, const float* dk_p_seed, const float* dv_p_seed,
                          void* dq_p, void* dk_p, void* dv_p, void* ws, size_t ws_bytes,
                          tree_attn_stream_t stream);

/*
 * Merge of partial attention states for the same query rows (section 3.3,
 * MoveQ, and Fig. 8: partial online-softmax states (m, l, O_acc) are merged
 * associatively, not normalised outputs).  A part is (O_k, LSE_k) with O_k
 * normalised; O_acc = l O and m = LSE - ln l carry the same information.
 *   LSE = ln sum_k exp(LSE_k),  O = sum_k exp(LSE_k - LSE) O_k.
 * A part with LSE_k = -inf (no visible key) is the identity; if every part
 * is empty the row gets LSE = -inf and O = 0.
 *   in : o_parts [num_splits, rows, heads, head_dim] float32,
 *        lse_parts [num_splits, heads, rows] float32
 *   out: o_out [rows, heads, head_dim] in out_dtype (a tree_attn_dtype),
 *        lse_out [heads, rows] float32
 * num_splits >= 1, rows >= 0, heads >= 1, head_dim in {64, 128}.
 */
int lse_merge(int32_t num_splits, int32_t rows, int32_t heads, int32_t head_dim,
              int32_t out_dtype, const float* o_parts, const float* lse_parts, void* o_out,
              float* lse_out, tree_attn_stream_t stream);

/*
 * The dQ strategy (TREE_ATTN_DQ_SEPARATE or TREE_ATTN_DQ_FUSED) that entry
 * point `op` (TREE_ATTN_OP_REPLAY_BWD or TREE_ATTN_OP_PREFILL_BWD) uses for
 * this problem: problem->dq_strategy when explicit, else the cost model's
 * choice.  Writes *strategy; no HIP call.  TREE_ATTN_ERR_INVALID for another
 * op; problem errors as tree_attn_workspace_size.
 */
int tree_attn_dq_strategy_of(const tree_attn_problem* problem, int op, int* strategy);

/*
 * How many chunks the replay query launch of entry point `op` cuts each
 * prompt column into for this problem (1 = not split): problem->
 * prompt_col_splits when set, else the makespan model's choice for that
 * launch.  op is TREE_ATTN_OP_REPLAY_FWD (the forward launch) or
 * TREE_ATTN_OP_REPLAY_BWD (the dQ launch of the separate strategy; 1 under
 * the fused strategy, which has none).  Writes *splits; no HIP call.
 */
int tree_attn_prompt_col_splits_of(const tree_attn_problem* problem, int op, int* splits);

/*
 * Work items the replay backward cuts the groups' prompt key tiles into,
 * per prompt tile position, summed over groups: n_g when no group is split,
 * more when some are (problem->prompt_tile_split_rows when set, else the
 * library's rule).  Writes *splits; no HIP call.
 */
int tree_attn_prompt_tile_splits_of(const tree_attn_problem* problem, int* splits);

/* A static description of a tree_attn_status code. */
const char* tree_attn_error_string(int code);

/*
 * Kernel timing hook for benchmarks and profilers.  kind 0 is the forward
 * attention kernel, 1 the dQ kernel, 2 the dK/dV kernel.  While set, every
 * launch of that kernel from the calling host thread records start_event
 * (a hipEvent_t) on the launch stream just before the kernel and
 * stop_event just after it; a later launch records them again.  NULL for
 * both events clears the hook.  Returns TREE_ATTN_ERR_INVALID for an
 * unknown kind or exactly one NULL event.  No HIP call.
 */
int tree_attn_set_kernel_events(int kind, void* start_event, void* stop_event);

/*
 * The hipError_t value behind the last TREE_ATTN_ERR_HIP returned on the
 * calling host thread (0 if none).  No HIP call.
 */
int tree_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H_ */
