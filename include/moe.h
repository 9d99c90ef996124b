/*
 * moe.h -- C ABI of libmoe: the MoE-layer hot path on one GPU's share of the
 * tokens, hand-written HIP kernels for gfx950 (MI355X).
 *
 * The calls follow the problem the pages pose:
 *  - route each token to k of E experts
 *      (Zyphra correlated expert placement page, English abstract);
 *  - count the expert pairs that one token activates together
 *      (Cobalt page, English abstract);
 *  - place E experts on G expert-parallel ranks and dispatch each token to
 *    each rank once, grouped by expert
 *      (Zyphra page, English abstract: correlated placement and the
 *       once-per-GPU dispatcher);
 *  - run the expert networks on the dispatched rows (same page);
 *  - combine the expert results back into token order (same page).
 *
 * Conventions shared by every call
 *  - Every pointer argument is DEVICE memory owned by the caller, except
 *    where a comment says otherwise. The library allocates nothing and keeps
 *    no state besides a per-device property cache.
 *  - Matrices are row-major and densely packed (row stride = row length).
 *  - bf16 tensors hold IEEE bfloat16 bit patterns (2 bytes per element).
 *  - Every call is asynchronous on `stream` (0 = the null stream) and only
 *    enqueues work; it never synchronises the host. Outputs must not alias
 *    inputs. Calls on disjoint buffers may run concurrently.
 *  - Argument errors are detected on the host before anything is enqueued
 *    and return MOE_ERR_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE with
 *    the outputs untouched. A failed kernel launch returns MOE_ERR_DEVICE.
 *  - VALUES inside device arrays cannot be seen by the host. The routing,
 *    co-activation and layout calls stay in bounds for any values: an expert
 *    id outside [0,E) or a rank outside [0,G) drops that choice (no slot, no
 *    row, slot_of -1), a repeated expert within a token or a NaN logit gives
 *    unspecified results. The expert, combine and backward calls trust the
 *    index arrays a layout call produced (perm_row, expert_off, slot_of);
 *    there a negative slot_of entry is a dropped choice that reads and adds
 *    nothing. moe_validate_routing checks routing inputs on the device.
 *  - Limits: 0 <= T, 1 <= k <= 16, k <= E <= 256, 1 <= G <= 32,
 *    T*k < 2^31. For the expert FFN d and F must be multiples of 64 and the
 *    FFN's tensors 16-byte aligned; in bf16 each call's activation operand
 *    (T*k rows) and each expert's weight matrix must be under 4 GiB - 4 KiB
 *    (else MOE_ERR_UNSUPPORTED).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef enum {
    MOE_OK = 0,
    MOE_ERR_ARG = 1,          /* a size, pointer or enum is invalid        */
    MOE_ERR_UNSUPPORTED = 2,  /* valid, but outside what the kernels cover */
    MOE_ERR_WORKSPACE = 3,    /* workspace missing or too small            */
    MOE_ERR_DEVICE = 4        /* a HIP call or kernel launch failed        */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Version of this ABI (MOE_ABI_VERSION of the build). */
int moe_abi_version(void);

/* Static string naming a status code. It takes an int, not a moe_status, so
   that any value (a code from a newer build, a corrupted one) gets a string:
   "unknown status" outside the enumeration. */
const char* moe_status_str(int status);

/*
 * Top-k routing (Zyphra page, English abstract: each token goes to k of the
 * E experts).
 *  logits   [T,E] fp32: router logits of T tokens.
 *  topk_idx [T,k] int32 out: chosen experts, by descending logit; equal
 *           logits go to the lower expert index (-0 equals +0).
 *  gates    [T,k] fp32 out: softmax over the k chosen logits (sums to 1).
 *  n_groups, topk_groups: group-limited routing. The E experts form n_groups
 *           contiguous groups of E/n_groups; a group's score is its largest
 *           logit; only the topk_groups best groups (ties -> lower group)
 *           stay eligible. n_groups = topk_groups = 1 is plain top-k.
 *           Requires n_groups | E, topk_groups <= n_groups and
 *           topk_groups * E / n_groups >= k.
 *  -inf logits are allowed as long as each token has k finite eligible ones.
 */
moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                     int32_t n_groups, int32_t topk_groups,
                     int32_t* topk_idx, float* gates, hipStream_t stream);

/*
 * Expert co-activation histogram (Cobalt page, English abstract: pairs of
 * experts that a single token activates together).
 *  topk_idx [T,k] int32: routing result (k distinct experts per token).
 *  coact    [E,E] int32 in/out: ACCUMULATES, for every token and every
 *           ordered pair (a,b), a != b, of its experts, coact[a][b] += 1.
 *           The matrix stays symmetric and its diagonal untouched; zero it
 *           first for a fresh count.
 */
moe_status moe_coact_hist(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                          int32_t* coact, hipStream_t stream);

/* Bytes of device workspace moe_dispatch_layout needs (host call, no GPU). */
size_t moe_dispatch_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t G);

/*
 * Dispatch layout and dispatch rows (Zyphra page, English abstract: experts
 * placed on GPUs, a dispatcher that sends each token to each GPU once).
 *  topk_idx  [T,k] int32: routing result.
 *  place     [E] int32: rank of each expert, in [0,G) (a partition).
 *  x         [T,d] activations (dt), or NULL to build only the indices.
 * Outputs (sized for the upper bound T*k where noted):
 *  rank_mask [T] uint32: bit g set iff a chosen expert of t sits on rank g.
 *  rank_off  [G+1] int32: row offsets per rank; R = rank_off[G] rows.
 *  disp_token[T*k] int32: first R entries: for each rank in order, the
 *            tokens sent to it in ascending order (one row per distinct
 *            (token, rank) pair).
 *  expert_off[E+1] int32: slot offsets per expert.
 *  perm_row  [T*k] int32: slot s (experts ascending, tokens ascending within
 *            an expert) reads dispatched row perm_row[s].
 *  slot_of   [T*k] int32: slot of (token t, choice j) at index t*k+j.
 *  x_disp    [T*k,d] (dt): rows 0..R-1 get x[disp_token[r]]; ignored if
 *            x is NULL.
 *  workspace: device scratch of at least moe_dispatch_workspace_bytes(),
 *            16-byte aligned, ZERO-FILLED before its first use: its first
 *            256 bytes hold a counter that the call's last count block uses
 *            and sets back to zero, so every call leaves it zero-filled.
 *            Calls that may run at the same time need separate workspaces.
 * R stays on the device; nothing is copied back to the host.
 */
moe_status moe_dispatch_layout(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                               const int32_t* place, int32_t G,
                               const void* x, int32_t d, moe_dtype dt,
                               uint32_t* rank_mask, int32_t* rank_off, int32_t* disp_token,
                               int32_t* expert_off, int32_t* perm_row, int32_t* slot_of,
                               void* x_disp, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * moe_dispatch_layout without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid allocation). Same arguments, outputs and orders as
 * moe_dispatch_layout. Its scratch is a library-owned device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU (held from the first call on that GPU
 * until the process ends); the call allocates nothing. Returns
 * MOE_ERR_WORKSPACE, enqueuing nothing, when the scratch the shape needs
 * (moe_dispatch_workspace_bytes(T, E, k, G)) exceeds that size; e.g.
 * T = 16384, E = 256, G = 32 needs 1.3 MB. The scratch starts zero-filled
 * (device memory of static storage) and every call leaves its counter word
 * at zero again, as moe_dispatch_layout requires of its workspace. Every
 * call on a GPU shares that GPU's scratch: calls that may overlap in time
 * on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_dispatch_layout_noalloc(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                                       const int32_t* place, int32_t G,
                                       const void* x, int32_t d, moe_dtype dt,
                                       uint32_t* rank_mask, int32_t* rank_off,
                                       int32_t* disp_token, int32_t* expert_off,
                                       int32_t* perm_row, int32_t* slot_of, void* x_disp,
                                       hipStream_t stream);

/*
 * Replica-aware dispatch layout (Cobalt page, English abstract: expert
 * replicas on GPUs of several nodes, and a communication-aware assignment
 * that routes each token to fewer remote nodes for the current layout).
 * Each chosen expert may have copies on several ranks; this call first picks
 * one rank per (token, choice), then builds the same once-per-rank layout as
 * moe_dispatch_layout from those ranks (outputs, orders and workspace are the
 * same; workspace size from moe_dispatch_workspace_bytes).
 *  rep_mask [E] uint32 (device): bit g set iff rank g holds a copy of expert
 *           e (bits >= G are ignored). Every expert a token chooses should
 *           have a copy: a choice without one is dropped (rank_of -1,
 *           slot_of -1, no slot and no row); the combine and backward
 *           calls leave it out (it has no expert output).
 *  ranks_per_node: ranks [n*rpn, (n+1)*rpn) form node n; rpn | G.
 * Assignment, per token t (home rank t*G/T, i.e. tokens sharded in order
 * over the ranks; home node = home rank / rpn), over its valid choices:
 *  nodes: while choices remain, take the node holding a copy of the most
 *         remaining choices (ties: the home node, then the lower node) and
 *         give it every remaining choice it can serve;
 *  ranks: inside each chosen node, in the order chosen, while its choices
 *         remain, take the node's rank holding the most of them (ties: the
 *         home rank, then the lower rank) and give it all it holds.
 * Extra outputs:
 *  rank_of   [T*k] int32: rank serving (t, j), or -1 if dropped.
 *  node_mask [T] uint32: bit n set iff a row of t goes to node n.
 * With one copy per expert (rep_mask[e] = 1 << place[e]) the layout equals
 * moe_dispatch_layout's.
 */
moe_status moe_replica_layout(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                              const uint32_t* rep_mask, int32_t G, int32_t ranks_per_node,
                              const void* x, int32_t d, moe_dtype dt, int32_t* rank_of,
                              uint32_t* node_mask, uint32_t* rank_mask, int32_t* rank_off,
                              int32_t* disp_token, int32_t* expert_off, int32_t* perm_row,
                              int32_t* slot_of, void* x_disp, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace moe_token_shuffle needs (host call, no GPU). */
size_t moe_shuffle_workspace_bytes(int32_t T, int32_t G);

/*
 * Token shuffling (Zyphra correlated expert placement page, English
 * abstract: under sequence parallelism each token is moved, during the
 * reduce-scatter after attention, to the GPU predicted to hold its
 * next-layer experts). The pages give no prediction rule; here the caller's
 * affinity table is the prediction model:
 *  want_idx [T,k] int32: the token's experts the prediction starts from
 *           (e.g. this layer's routing); entries outside [0,E) add nothing.
 *  aff      [E,G] int32: aff[e][g] = how strongly a token using expert e is
 *           expected to need rank g next (e.g. cross-layer co-activation
 *           counts summed over the next layer's experts on g; the one-hot
 *           table of a placement gives "the rank holding most of them").
 * Destination of token t: the rank g maximising sum_j aff[want[t,j]][g]
 * (int64 sums; ties: the home rank t*G/T, then the lowest rank).
 * Outputs:
 *  dest     [T] int32: destination rank of each token.
 *  rank_off [G+1] int32: token offsets per rank in the shuffled order.
 *  perm     [T] int32: tokens in shuffled order (grouped by destination,
 *           ascending within a rank).
 *  pos      [T] int32: position of token t in that order (perm[pos[t]] = t).
 *  x_shuf   [T,d] (dt): x[perm[i]] in row i; ignored if x is NULL.
 *  workspace: device scratch of at least moe_shuffle_workspace_bytes(),
 *           16-byte aligned and zero-filled before its first use, as for
 *           moe_dispatch_layout (every call leaves it so).
 * G <= 32, k <= 16.
 */
moe_status moe_token_shuffle(const int32_t* want_idx, int32_t T, int32_t E, int32_t k,
                             const int32_t* aff, int32_t G, const void* x, int32_t d,
                             moe_dtype dt, int32_t* dest, int32_t* rank_off, int32_t* perm,
                             int32_t* pos, void* x_shuf, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Bytes of device workspace the forward expert calls need (host call, no
 * GPU): the tile queue of their persistent launches. */
size_t moe_expert_workspace_bytes(void);

/*
 * Expert networks, first half: for every slot s of expert e (expert_off),
 *   a = x_disp[perm_row[s]],  u = W_gate[e] a,  v = W_up[e] a,
 *   h[s] = silu(u) * v,       silu(u) = u / (1 + exp(-u)).
 * The pages only say "expert networks"; this is a bias-free SwiGLU MLP.
 *  x_disp [*,d] (dt), w_gate / w_up [E,F,d] (dt, output index first),
 *  h [T*k,F] (dt) out; rows expert_off[E]..T*k-1 are not written.
 *  workspace: at least moe_expert_workspace_bytes() bytes, 16-byte aligned,
 *  ZERO-FILLED before its first use; every call leaves it zero-filled again
 *  (it holds the tile queue of the persistent launch, which the launch's
 *  last workgroup resets). Calls that may run at the same time (other
 *  streams) need separate workspaces. Missing or small: MOE_ERR_WORKSPACE.
 * bf16: bf16 MFMA with fp32 accumulation, h rounded to bf16 (RNE).
 */
moe_status moe_expert_gate_up(const void* x_disp, const int32_t* perm_row,
                              const int32_t* expert_off, int32_t T, int32_t E, int32_t k,
                              int32_t d, int32_t F, const void* w_gate, const void* w_up,
                              moe_dtype dt, void* h, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Expert networks, second half: y[s] = W_down[e] h[s] for every slot s of
 * expert e.  h [T*k,F] (dt), w_down [E,d,F] (dt), y [T*k,d] (dt) out.
 * workspace as for moe_expert_gate_up.
 */
moe_status moe_expert_down(const void* h, const int32_t* expert_off, int32_t T, int32_t E,
                           int32_t k, int32_t d, int32_t F, const void* w_down, moe_dtype dt,
                           void* y, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Both halves in order: moe_expert_gate_up then moe_expert_down (one
 * workspace serves both: the second launch starts after the first has
 * reset it). */
moe_status moe_grouped_ffn(const void* x_disp, const int32_t* perm_row, const int32_t* expert_off,
                           int32_t T, int32_t E, int32_t k, int32_t d, int32_t F,
                           const void* w_gate, const void* w_up, const void* w_down, moe_dtype dt,
                           void* h, void* y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Combine back to token order (Zyphra page, English abstract: the expert
 * results are combined): out[t] = sum_j gates[t,j] * y[slot_of[t*k+j]],
 * accumulated in fp32 in j order, stored in dt (bf16: RNE).
 *  y [T*k,d] (dt), slot_of [T*k], gates [T,k] fp32 (NULL: every gate is
 *  1), out [T,d] (dt) out. A choice with slot_of < 0 (dropped by
 *  moe_replica_layout) is left out of the sum and no y row is read for it.
 */
moe_status moe_combine(const void* y, const int32_t* slot_of, const float* gates,
                       int32_t T, int32_t k, int32_t d, moe_dtype dt, void* out,
                       hipStream_t stream);

/*
 * ---- Backward pass (training). The pages train these layers: expert
 * parallelism runs its all-to-all in the forward and the backward pass
 * (Zyphra correlated expert placement page, English abstract). Each call is
 * the exact gradient of the matching forward step for a loss whose gradient
 * at the layer output is dout; weight gradients are written (not added) in
 * fp32, activation gradients in dt. Slots, offsets and permutations are
 * those of the forward's layout.
 */

/* Forward gate/up that also keeps the pre-activations for the backward:
 * uv [T*k, 2F] (dt): row s = [u_s | v_s] (u = W_gate a, v = W_up a).
 * workspace as for moe_expert_gate_up. */
moe_status moe_expert_gate_up_save(const void* x_disp, const int32_t* perm_row,
                                   const int32_t* expert_off, int32_t T, int32_t E, int32_t k,
                                   int32_t d, int32_t F, const void* w_gate, const void* w_up,
                                   moe_dtype dt, void* h, void* uv, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Combine backward: dy[slot_of[t*k+j]] = gates[t,j] * dout[t] (dt) and
 * dgates[t,j] = <dout[t], y[slot_of[t*k+j]]> (fp32 accumulation).
 *  dout [T,d], y [T*k,d], dy [T*k,d] (dt); gates, dgates [T,k] fp32.
 *  A dropped choice (slot_of < 0) writes no dy row and gets dgates 0. */
moe_status moe_combine_bwd(const void* dout, const void* y, const int32_t* slot_of,
                           const float* gates, int32_t T, int32_t k, int32_t d, moe_dtype dt,
                           void* dy, float* dgates, hipStream_t stream);

/* Bytes of device workspace moe_expert_down_bwd and moe_expert_gate_up_bwd
 * need (host call, no GPU): in bf16 the weight gradients transpose their
 * second operand (h, or the gathered a) into expert-padded K-contiguous rows
 * there and keep the persistent launch's tile queue (about
 * max(F, d) * (T*k + 64 E) * 2 bytes). */
size_t moe_expert_bwd_workspace_bytes(int32_t T, int32_t E, int32_t k, int32_t d, int32_t F);

/* Down projection and SwiGLU backward, per expert e over its slots s:
 *  dh = dy[s] W_down[e];  du = dh * v * silu'(u),  dv = dh * silu(u)
 *  (silu'(u) = sg (1 + u (1 - sg)), sg = 1 / (1 + e^-u); u, v from uv);
 *  duv [T*k, 2F] (dt) out: row s = [du_s | dv_s];
 *  dw_down [E,d,F] fp32 out: dw_down[e] = sum_s dy[s] h[s]^T (zero for an
 *  expert without slots). h [T*k,F], uv [T*k,2F], w_down [E,d,F] (dt).
 *  workspace: device scratch of at least moe_expert_bwd_workspace_bytes()
 *  (bf16; may be NULL for fp32). */
moe_status moe_expert_down_bwd(const void* dy, const void* h, const void* uv,
                               const int32_t* expert_off, int32_t T, int32_t E, int32_t k,
                               int32_t d, int32_t F, const void* w_down, moe_dtype dt, void* duv,
                               float* dw_down, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Gate/up backward, per expert e over its slots s (a_s = x_disp[perm_row[s]]):
 *  da [T*k,d] (dt) out: da[s] = du_s W_gate[e] + dv_s W_up[e];
 *  dw_gate, dw_up [E,F,d] fp32 out: sum_s du_s a_s^T and sum_s dv_s a_s^T.
 *  x_disp has T*k rows of capacity. workspace as for moe_expert_down_bwd. */
moe_status moe_expert_gate_up_bwd(const void* duv, const void* x_disp, const int32_t* perm_row,
                                  const int32_t* expert_off, int32_t T, int32_t E, int32_t k,
                                  int32_t d, int32_t F, const void* w_gate, const void* w_up,
                                  moe_dtype dt, void* da, float* dw_gate, float* dw_up,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dispatch backward: dx[t] = sum_j da[slot_of[t*k+j]] (fp32 accumulation in
 * j order, stored in dt) over the choices with slot_of >= 0.
 * da [T*k,d], dx [T,d]. */
moe_status moe_dispatch_bwd(const void* da, const int32_t* slot_of, int32_t T, int32_t k,
                            int32_t d, moe_dtype dt, void* dx, hipStream_t stream);

/* Routing backward (softmax over the chosen logits):
 *  dlogits[t, topk_idx[t,j]] = g_j (dg_j - sum_i g_i dg_i), every other
 *  entry 0. gates, dgates [T,k] fp32, dlogits [T,E] fp32 out. E <= 1024. */
moe_status moe_route_bwd(const float* gates, const float* dgates, const int32_t* topk_idx,
                         int32_t T, int32_t E, int32_t k, float* dlogits, hipStream_t stream);

/*
 * Device-side validation of routing inputs, for debugging (the binding runs
 * it after routing when MOE_DEBUG=1 is set). Each check covers a value the
 * host cannot see and the other calls do not define:
 *  logits   [T,E] fp32 (or NULL): a NaN logit has no place in the descending
 *           order of logits (Zyphra page, English abstract: each token goes
 *           to k of the E experts)                      -> MOE_BAD_LOGIT;
 *  topk_idx [T,k] int32 (or NULL): each entry in [0,E)  -> MOE_BAD_EXPERT,
 *           and the k entries of a token distinct       -> MOE_BAD_REPEAT;
 *  place    [E] int32 (or NULL): each rank in [0,G)     -> MOE_BAD_RANK.
 *  err      [1] uint32 in/out: the flags found are OR-ed in; zero it first.
 * Asynchronous like every call: read err after synchronising the stream.
 * k <= 16. Nothing traps; the kernel reads every value once.
 */
enum {
    MOE_BAD_LOGIT = 1u,
    MOE_BAD_EXPERT = 2u,
    MOE_BAD_REPEAT = 4u,
    MOE_BAD_RANK = 8u
};
moe_status moe_validate_routing(const float* logits, const int32_t* topk_idx, int32_t T,
                                int32_t E, int32_t k, const int32_t* place, int32_t G,
                                uint32_t* err, hipStream_t stream);

/*
 * Expert placement planner (host code; every pointer is HOST memory).
 * Cobalt page, English abstract: a two-stage layout planner that co-locates
 * frequently co-activated experts and rebalances the workload inside each
 * node; Zyphra page, English abstract: experts selected together go to the
 * same GPU, so the once-per-GPU dispatcher sends fewer rows.
 *  coact  [E,E] int64: co-activation counts (e.g. moe_coact_hist summed over
 *         steps); weights are coact[a][b] + coact[b][a], the diagonal is
 *         ignored. Must be >= 0.
 *  load   [E] int64: per-expert token counts (>= 0), e.g. expert_off deltas.
 *  G ranks with E/G experts each (G | E); ranks_per_node | G groups ranks
 *         [n*rpn, (n+1)*rpn) into node n.
 *  Stage 1: for each rank in turn, seed with the heaviest unassigned expert
 *         and add the unassigned expert with the most co-activation weight
 *         to the rank's members until it holds E/G; then up to swap_passes
 *         passes over expert pairs (a < b) in different ranks, swapping
 *         whenever that raises the total within-rank weight.
 *  Stage 2 (ranks_per_node > 1): inside each node, repeatedly apply the
 *         swap between its most and least loaded ranks that most lowers the
 *         larger of their two loads (ties: most within-rank weight kept)
 *         while it lowers it. Experts stay in their node.
 *  Ties go to the lower expert / rank index (deterministic).
 *  place  [E] int32 out: rank of each expert.
 * Limits: E <= 256, G <= 32. Bad sizes or negative counts: MOE_ERR_ARG.
 * Runs on the calling thread; no GPU work.
 */
moe_status moe_plan_placement(const int64_t* coact, const int64_t* load, int32_t E, int32_t G,
                              int32_t ranks_per_node, int32_t swap_passes, int32_t* place);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
