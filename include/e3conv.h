/*
 * e3conv -- equivariant message-passing convolution on AMD MI355X (gfx950).
 *
 * The operation (e3j Convolution API page: the class formula, and the
 * unfused JAX implementation described beneath it):
 *
 *     out[b] = (1/N) * sum over edges e = (a -> b) of  (x[a] (x) y[e]) (.) s[e]
 *
 * - x  node features, shape (num_nodes, num_x, C), trailing channel axis
 *      ("TRAILING_CHANNELS" layout of that page);
 * - y  edge features (spherical harmonics 0..sh_lmax), shape (num_edges, num_y),
 *      no channel axis, broadcast over channels;
 * - s  edge scalars, shape (num_edges, num_paths, C): one value per
 *      (path, channel); the page derives this space from those of x and y;
 * - (x) the channelwise Clebsch-Gordan tensor product, one path per allowed
 *      (x block, l2, output block) triple; (.) the per-(path, channel) mixing;
 * - the sum runs over the incoming edges of receiver b (RECEIVER ordering of
 *      that page: edges sorted by receiver, so aggregation is a segmented sum);
 * - N = avg_num_neighbors: every message is scaled by 1/N.
 *
 * Conventions (readings of the pages; the pages print no formula for them):
 * - components: blocks in the order given, m = -l..l inside a block, real
 *   spherical-harmonic basis with z as polar axis (l=1 is (y, z, x));
 * - a path (l1,p1) x l2 -> (l3,p3) exists iff |l1-l2| <= l3 <= l1+l2 and
 *   p3 = p1 (-1)^l2; paths are ordered x block, then l2 = 0..sh_lmax, then
 *   output block, which is the order of the s scalar axis;
 * - the CG tensor of each path is the real, orthonormal one
 *   (sum_{m1,m2} C[m1,m2,m3] C[m1,m2,m3'] = delta), sign fixed so that its first
 *   nonzero entry in (m1, m2, m3) order is positive ("SQRT_DIM_OUT"
 *   normalization named on the e3j page);
 * - paths into the same output block add up.
 *
 * Memory and streams: every device pointer is owned by the caller; no compute
 * call allocates device memory (only the synchronous checking convenience
 * e3conv_validate_graph(on_device = 1) does).  Tensors are dense, row-major, at least
 * 16-byte aligned.  Indices are int32.  All device work is enqueued on the
 * caller's hipStream_t (passed as void*), asynchronously, with no implicit
 * synchronisation.  Errors are reported by status code; a human-readable
 * message for the last error on the calling thread is available from
 * e3conv_last_error_detail().  No C++ exception crosses this boundary.
 */
#ifndef E3CONV_H
#define E3CONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct e3conv_plan_s* e3conv_plan_t;

typedef enum {
  E3CONV_OK = 0,
  E3CONV_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad dtype */
  E3CONV_ERR_PARSE = 2,            /* malformed irreps string                 */
  E3CONV_ERR_UNSUPPORTED = 3,      /* no compiled kernel for this layout/dtype */
  E3CONV_ERR_NO_PATH = 4,          /* an output block is reached by no path   */
  E3CONV_ERR_GRAPH = 5,            /* graph failed validation                 */
  E3CONV_ERR_WORKSPACE = 6,        /* workspace too small                     */
  E3CONV_ERR_HIP = 7,              /* a HIP runtime call or launch failed     */
  E3CONV_ERR_INTERNAL = 8          /* host CG table disagrees with the kernel pattern */
} e3conv_status;

typedef enum { E3CONV_F32 = 0, E3CONV_BF16 = 1 } e3conv_dtype;

/* Graph ordering (e3j Convolution page, graph_ordering parameter and its note
 * on the fused kernels).  RECEIVER: edges grouped by receiver; out[b] sums
 * the incoming edges of b directly.  SENDER: edges grouped by sender; out[b]
 * is assembled from the outgoing edges e = (b -> a) of b as
 * (1/N) sum_e (x[a] (x) P y[e]) (.) s[e], where P negates the odd-l blocks of
 * y.  Under the page's assumptions for SENDER ordering (the graph holds b->a
 * whenever it holds a->b, y[b->a] = (-1)^l y[a->b] per l block, and
 * s[b->a] = s[a->b]) this
 * equals the RECEIVER result; the library computes the formula above
 * whether or not they hold, and its reverse pass is the exact derivative of
 * that formula. */
typedef enum { E3CONV_RECEIVER = 0, E3CONV_SENDER = 1 } e3conv_ordering;

/* Build a plan (host only, no device call).
 *   irreps_in   x irreps, e.g. "128x0e+128x1o" or "64x(0e+1o+2e)"; every block
 *               must have the same multiplicity C (the channel count);
 *   sh_lmax     edge features are spherical harmonics l = 0..sh_lmax (num_y =
 *               (sh_lmax+1)^2), 0 <= sh_lmax <= 6;
 *   irreps_out  output irreps (same multiplicity C); acts as the filter on
 *               output blocks ("target" on the e3j page);
 *   avg_num_neighbors  N > 0; pass 1 for no rescaling.
 * Irreps have l <= 6.  Duplicate irreps, mixed multiplicities and output blocks
 * no path reaches are rejected.  A plan whose layout has no compiled kernel is
 * still created (its tables can be queried); e3conv_forward/_backward then
 * return E3CONV_ERR_UNSUPPORTED.  On success *plan_out owns the plan; free it
 * with e3conv_plan_destroy.  Plans are immutable and thread-safe. */
e3conv_status e3conv_plan(const char* irreps_in, int sh_lmax, const char* irreps_out,
                          float avg_num_neighbors, e3conv_plan_t* plan_out);

/* As e3conv_plan, with the graph ordering chosen explicitly (e3conv_plan is
 * RECEIVER).  For a SENDER plan every call takes, in place of the receiver
 * CSR and the senders, the sender CSR (row_ptr: edges of sender b are
 * row_ptr[b] .. row_ptr[b+1]-1) and src[e] = the receiver of edge e, the node
 * whose features are gathered; the y, s, grad_y and grad_s rows follow that
 * edge order.  E3CONV_ERR_INVALID_ARGUMENT for another ordering value. */
e3conv_status e3conv_plan_ordered(const char* irreps_in, int sh_lmax, const char* irreps_out,
                                  float avg_num_neighbors, e3conv_ordering ordering,
                                  e3conv_plan_t* plan_out);

/* The plan's graph ordering. */
e3conv_status e3conv_plan_ordering(e3conv_plan_t plan, e3conv_ordering* ordering);

void e3conv_plan_destroy(e3conv_plan_t plan);

/* Per-channel sizes of the operands: x (N, num_x, C), y (E, num_y),
 * s (E, num_paths, C), out (N, num_out, C).  Any pointer may be NULL. */
e3conv_status e3conv_plan_shape(e3conv_plan_t plan, int* channels, int* num_x, int* num_y,
                                int* num_paths, int* num_out);

/* Path table, one entry per path in s-axis order: l and parity of the x block,
 * l2 of the edge harmonic, l and parity of the output block, and the component
 * offsets of the three blocks.  Each array has num_paths entries; any may be NULL. */
e3conv_status e3conv_plan_paths(e3conv_plan_t plan, int* l1, int* p1, int* l2, int* l3,
                                int* p3, int* o1, int* o2, int* o3);

/* Packed coefficients (the e3j "coef" attribute read as a sparse 4-index list):
 * out[b, iout, c] += value * x[a, ix, c] * y[e, iy] * s[e, ip, c] / N.
 * Call with NULL arrays to get *nnz; then call again with arrays of *nnz
 * entries.  Entries are the nonzero real CG values in fp64. */
e3conv_status e3conv_plan_coefficients(e3conv_plan_t plan, int* nnz, int* ix, int* iy,
                                       int* ip, int* iout, double* value);

/* Whether compiled kernels exist for this plan: forward for f32 and bf16
 * inputs, backward (f32).  Any pointer may be NULL. */
e3conv_status e3conv_plan_supported(e3conv_plan_t plan, int* fwd_f32, int* fwd_bf16, int* bwd_f32);

/* Forward convolution.
 *   in_dtype  storage type of x, y and s (E3CONV_F32 or E3CONV_BF16: bf16 is
 *             read as raw 16-bit words); accumulation and out are fp32;
 *   x, y, s   device pointers, shapes above;
 *   src       device int32[num_edges]: sender of each edge, in [0, num_nodes);
 *   row_ptr   device int32[num_nodes + 1]: receiver CSR offsets, row_ptr[0] = 0,
 *             row_ptr[num_nodes] = num_edges; edges of receiver b are
 *             row_ptr[b] .. row_ptr[b+1]-1 (y and s rows in that order);
 *   order     device int32[num_nodes], a permutation of 0..num_nodes-1 giving
 *             the order in which receivers are processed (for cache reuse of
 *             the gathered sender rows, see e3conv_receiver_order), or NULL
 *             for 0..num_nodes-1.  The result does not depend on it (bitwise);
 *   out       device float[num_nodes * num_out * C], fully overwritten (rows of
 *             receivers without edges are set to zero);
 *   hip_stream  hipStream_t or NULL for the default stream.
 * Indices out of range or a non-monotone row_ptr are undefined behaviour (the
 * fused kernels need sorted edges, as on the e3j page); check them once per
 * graph with e3conv_validate_graph.  num_edges = 0 is valid (out is zeroed);
 * num_nodes = 0 is a no-op.  Sizes must satisfy num_edges < 2^31 and
 * num_nodes * num_out * C < 2^31. */
e3conv_status e3conv_forward(e3conv_plan_t plan, e3conv_dtype in_dtype, const void* x,
                             const void* y, const void* s, const int32_t* src,
                             const int32_t* row_ptr, const int32_t* order, int64_t num_nodes,
                             int64_t num_edges, float* out, void* hip_stream);

/* Forward with padding nodes (e3j Convolution page, node_mask argument: True
 * for real nodes, False for padding nodes, which lie at the tail; padding
 * edges only connect padding nodes).  The mask is given as its count of real
 * nodes: nodes num_real_nodes .. num_nodes-1 are padding.  Rows of padding
 * nodes are set to zero and their edges are not read; real rows equal
 * e3conv_forward's.  0 <= num_real_nodes <= num_nodes, else
 * E3CONV_ERR_INVALID_ARGUMENT.  Other arguments as e3conv_forward (the
 * unmasked call is num_real_nodes = num_nodes). */
e3conv_status e3conv_forward_masked(e3conv_plan_t plan, e3conv_dtype in_dtype, const void* x,
                                    const void* y, const void* s, const int32_t* src,
                                    const int32_t* row_ptr, const int32_t* order,
                                    int64_t num_nodes, int64_t num_edges, int64_t num_real_nodes,
                                    float* out, void* hip_stream);

/* Convolution with the edge scalars computed from the edge lengths in the
 * kernel (e3nn_mlx gate-points page: radial embedding of each edge length and
 * the fully connected network that maps it to the convolution's per-path,
 * per-channel weights; the network's two weight layers without biases):
 *     f_k(r) = exp(-((r - mu_k) / sigma)^2) * (1 + cos(pi r / r_max)) / 2 for r < r_max,
 *              0 for r >= r_max (the cosine cutoff vanishes from r_max on),
 *              mu_k = k r_max / (num_basis - 1),
 *     s[e]   = silu(f(r[e]) w1) w2, reshaped (num_paths, C), silu(z) = z / (1 + e^-z),
 * then out as e3conv_forward.  The scalars are formed per receiver in
 * registers and never written to memory.
 * - x (num_nodes, num_x, C), y (num_edges, num_y), r (num_edges): fp32 device,
 *   edges sorted by receiver as in e3conv_forward; out fp32 (num_nodes,
 *   num_out, C), fully overwritten.
 * - w1 (num_basis, hidden), w2 (hidden, num_paths * C): fp32 device, row
 *   major; column p * C + c of w2 produces s[., p, c].
 * - 2 <= num_basis <= 8; hidden a multiple of 4 in [4, 128]; r_max, sigma > 0,
 *   else E3CONV_ERR_INVALID_ARGUMENT.  Edges with r >= r_max may be present:
 *   their scalars, and so their messages, are zero.
 * - Compiled for layouts of 32 channels and at most 8 paths (the gate-points
 *   layout) in RECEIVER ordering; other plans give E3CONV_ERR_UNSUPPORTED.
 * - order and num_real_nodes as e3conv_forward_masked.
 * - Arithmetic: fp32 inputs and outputs at fp32-level accuracy.  The second
 *   layer's products run as three fp16 matrix products of operands split in
 *   two fp16 parts, with power-of-two scales chosen from the weights that keep
 *   every operand inside the fp16 range. */
e3conv_status e3conv_forward_radial(e3conv_plan_t plan, const float* x, const float* y, const float* r,
                                    const float* w1, const float* w2, int32_t num_basis,
                                    int32_t hidden, float r_max, float sigma, const int32_t* src,
                                    const int32_t* row_ptr, const int32_t* order, int64_t num_nodes,
                                    int64_t num_edges, int64_t num_real_nodes, float* out,
                                    void* hip_stream);

/* Forward-mode derivative (Jacobian-vector product; e3nn_mlx page, "JVP and
 * generated-kernel boundary").  The convolution is trilinear, so along the
 * tangent (dx, dy, ds)
 *     out_dot = conv(dx, y, s) + conv(x, dy, s) + conv(x, y, ds),
 * computed in one pass that also yields out = conv(x, y, s).  dx, dy, ds have
 * the shapes and in_dtype of x, y, s; out (may be NULL when not wanted) and
 * out_dot are fp32 (num_nodes, num_out, C), fully overwritten.  Graph
 * arguments, ordering, node-mask count and rules as e3conv_forward_masked
 * (num_real_nodes = num_nodes for no padding). */
e3conv_status e3conv_jvp(e3conv_plan_t plan, e3conv_dtype in_dtype, const void* x, const void* y,
                         const void* s, const void* dx, const void* dy, const void* ds,
                         const int32_t* src, const int32_t* row_ptr, const int32_t* order,
                         int64_t num_nodes, int64_t num_edges, int64_t num_real_nodes, float* out,
                         float* out_dot, void* hip_stream);

/* Bytes of device workspace e3conv_backward needs (currently 0). */
e3conv_status e3conv_backward_workspace_size(e3conv_plan_t plan, int64_t num_nodes,
                                             int64_t num_edges, size_t* bytes);

/* Reverse pass of L = <grad_out, out> (fp32 only): given grad_out (N, num_out, C)
 * writes grad_x (N, num_x, C), grad_y (E, num_y) and grad_s (E, num_paths, C).
 * Same graph arguments and rules as e3conv_forward.  grad_x is fully
 * overwritten (zeroed, then accumulated across the edges leaving each node with
 * fp32 device atomics, so its rounding may vary from run to run); grad_y and
 * grad_s are written once per edge.  If grad_x, grad_y and grad_s are all
 * NULL the call does nothing; otherwise grad_x and grad_out are required, and
 * grad_y, grad_s, x, y, s and src are required when num_edges > 0 (they may
 * be NULL for an edgeless graph).  workspace may be NULL when the size is 0. */
e3conv_status e3conv_backward(e3conv_plan_t plan, e3conv_dtype in_dtype, const void* x,
                              const void* y, const void* s, const int32_t* src,
                              const int32_t* row_ptr, const int32_t* order, int64_t num_nodes,
                              int64_t num_edges, const float* grad_out, float* grad_x,
                              float* grad_y,
                              float* grad_s, void* workspace, size_t workspace_bytes,
                              void* hip_stream);

/* Flags of e3conv_backward_ex: add the gradient into the caller's array
 * instead of overwriting it. */
#define E3CONV_ACCUMULATE_GRAD_X 1u
#define E3CONV_ACCUMULATE_GRAD_Y 2u
#define E3CONV_ACCUMULATE_GRAD_S 4u

/* General reverse pass: e3conv_backward with node-mask padding (edges of
 * receivers b >= num_real_nodes contribute nothing: zero grad_y and grad_s
 * rows, nothing added to grad_x; the derivative of e3conv_forward_masked),
 * optional outputs (any of grad_x, grad_y, grad_s may be NULL: not
 * computed; all NULL is a no-op) and accumulation (flags: a set
 * E3CONV_ACCUMULATE_GRAD_* bit adds into that array, which must then hold
 * valid data; otherwise it is overwritten).  Unknown flag bits are
 * E3CONV_ERR_INVALID_ARGUMENT.  These are the building blocks of second
 * derivatives (reverse over reverse), where the gradient of <G, grad> with
 * respect to each operand sums reverse passes with one operand replaced by a
 * cotangent.  With flags = 0 and all three outputs it runs the same kernels as
 * e3conv_backward. */
e3conv_status e3conv_backward_ex(e3conv_plan_t plan, e3conv_dtype in_dtype, const void* x,
                                 const void* y, const void* s, const int32_t* src,
                                 const int32_t* row_ptr, const int32_t* order, int64_t num_nodes,
                                 int64_t num_edges, int64_t num_real_nodes, const float* grad_out,
                                 float* grad_x, float* grad_y, float* grad_s, unsigned flags,
                                 void* workspace, size_t workspace_bytes, void* hip_stream);

/* Second derivatives of the training step (e3nn_mlx page: reverse over
 * reverse).  With (grad_x, grad_y, grad_s) the reverse pass of L = <grad_out,
 * out> at (x, y, s), and cotangents (cot_x, cot_y, cot_s) of those gradients,
 * this writes the gradient of L2 = <cot_x, grad_x> + <cot_y, grad_y> +
 * <cot_s, grad_s> with respect to x, y, s and grad_out:
 *     d_x  = reverse(x, cot_y, s).grad_x + reverse(x, y, cot_s).grad_x,
 *     d_y  = reverse(cot_x, y, s).grad_y + reverse(x, y, cot_s).grad_y,
 *     d_s  = reverse(cot_x, y, s).grad_s + reverse(x, cot_y, s).grad_s,
 *     d_grad_out = forward-mode derivative of out along (cot_x, cot_y, cot_s)
 * (L2 = <grad_out, D out(x, y, s)[cot_x, cot_y, cot_s]>, and out is trilinear).
 * Three general reverse passes and one forward-mode pass, enqueued on
 * hip_stream; fp32 only.  Every array has the shape of its namesake (d_x and
 * cot_x as x, d_grad_out as grad_out, ...); the outputs are overwritten.
 * Graph arguments and num_real_nodes as e3conv_backward_ex. */
e3conv_status e3conv_second_derivatives(e3conv_plan_t plan, e3conv_dtype in_dtype, const void* x,
                                        const void* y, const void* s, const int32_t* src,
                                        const int32_t* row_ptr, const int32_t* order,
                                        int64_t num_nodes, int64_t num_edges,
                                        int64_t num_real_nodes, const float* grad_out,
                                        const float* cot_x, const float* cot_y,
                                        const float* cot_s, float* d_x, float* d_y, float* d_s,
                                        float* d_grad_out, void* hip_stream);

/* Pair-stored reverse pass (e3j Convolution page, the note on SENDER
 * ordering, which assumes a symmetric graph, y_ba = (-1)^l y_ab per l block and
 * s_ba = s_ab).  Under those assumptions one row of y and s per undirected
 * pair carries the whole graph: a stored edge e = (a -> b), a = src[e],
 * b = dst[e], stands for itself, with y[e] and s[e], and for its reverse
 * (b -> a), with P y[e] (odd-l blocks negated) and s[e].  The forward
 * function is the RECEIVER convolution (formula above) of those 2 E directed
 * edges, and this call is its reverse pass for L = <grad_out, out>:
 *     grad_s[e] = ds(a -> b) + ds(b -> a),
 *     grad_y[e] = dy(a -> b) + P dy(b -> a),
 *     grad_x    = the sum over all 2 E directed edges, as in e3conv_backward.
 * s[e] is read and grad_s[e] written once per pair, which halves the edge
 * bytes of the directed reverse pass on the same graph.
 *   x (N, num_x, C), y (E, num_y), s (E, num_paths, C), grad_out (N, num_out,
 *   C): fp32 device; src, dst: device int32[E] in [0, num_nodes) (out of range
 *   is undefined behaviour); E = num_pairs;
 *   grad_x (N, num_x, C): fully overwritten (zeroed, then fp32 atomics, so its
 *   rounding may vary from run to run); grad_y (E, num_y) and grad_s (E,
 *   num_paths, C) written once per stored edge.
 * The stored edges may come in any order with either orientation (a pair
 * stored as (b -> a) with P y gives the same grad_x and grad_s, and P grad_y);
 * grouping the edges with equal dst consecutively (e.g. sorted by dst) lets
 * each run share one set of grad_x[b] atomics.  A stored self loop (a = b)
 * counts as two edges.  RECEIVER plans only (E3CONV_ERR_UNSUPPORTED
 * otherwise, or for a layout without this kernel); num_nodes = 0 with
 * num_pairs = 0 is a no-op; asynchronous on hip_stream. */
e3conv_status e3conv_backward_pairs(e3conv_plan_t plan, const float* x, const float* y,
                                    const float* s, const int32_t* src, const int32_t* dst,
                                    int64_t num_nodes, int64_t num_pairs, const float* grad_out,
                                    float* grad_x, float* grad_y, float* grad_s, void* hip_stream);

/* Output linear: channel mixing within each output irrep block, the step
 * after the convolution (cuEquivariance page, Flax NNX layers, IrrepsLinear:
 * each block is mixed across its channels by a weight matrix and scaled by
 * scale / sqrt of the input multiplicity).  For every output block k of the plan, with C = the plan's
 * channels and C_out = channels_out,
 *     out[b, i, v] = scale / sqrt(C) * sum_u weights[k, u, v] * in[b, i, u]
 * for each component i of block k.
 *   weights  device float[num_out_blocks * C * C_out] (blocks in the plan's
 *            output order, then u, then v);
 *   in       device float (num_nodes, num_out, C), e.g. e3conv_forward's out;
 *   out      device float (num_nodes, num_out, C_out), fully overwritten.
 * fp32 products at fp32 accuracy and fp32 sums on the matrix cores (each
 * operand split into three bf16 parts, six partial products per product);
 * asynchronous on hip_stream.
 * channels_out > 0, scale finite, num_out <= 128 components, else
 * E3CONV_ERR_INVALID_ARGUMENT / E3CONV_ERR_UNSUPPORTED. */
e3conv_status e3conv_linear(e3conv_plan_t plan, int channels_out, float scale,
                            const float* weights, const float* in, int64_t num_nodes, float* out,
                            void* hip_stream);

/* The convolution with the output linear fused into its epilogue: out =
 * e3conv_linear(plan, C, scale, weights, e3conv_forward(...)) with
 * channels_out = C, in one pass (cuEquivariance page, Flax NNX layers,
 * IrrepsLinear, applied to the convolution's output).  Each receiver's row is
 * mixed per output irrep block by the C x C weight block while still on chip,
 * so the convolution's own output never reaches memory.  Arguments as
 * e3conv_forward (x, y, s in in_dtype; out fp32 (num_nodes, num_out, C),
 * fully overwritten) plus scale (finite) and weights (device float[
 * num_out_blocks * C * C], blocks in the plan's output order, then u, then v,
 * as e3conv_linear).  Compiled for RECEIVER plans of up to 64 channels, whose
 * weight blocks fit one work-group's LDS (at most 64 KiB); other plans give
 * E3CONV_ERR_UNSUPPORTED (use e3conv_forward, then e3conv_linear).  fp32
 * products on the vector ALU; asynchronous on hip_stream. */
e3conv_status e3conv_forward_linear(e3conv_plan_t plan, e3conv_dtype in_dtype, const void* x,
                                    const void* y, const void* s, const int32_t* src,
                                    const int32_t* row_ptr, const int32_t* order,
                                    int64_t num_nodes, int64_t num_edges, float scale,
                                    const float* weights, float* out, void* hip_stream);

/* Reverse pass of e3conv_linear for L = <grad_out, out>:
 *   grad_in[b, i, u]   = scale / sqrt(C) * sum_v weights[k, u, v] grad_out[b, i, v]
 *   grad_weights[k, u, v] = scale / sqrt(C) * sum_{b, i in block k} in[b, i, u] grad_out[b, i, v]
 * Either output may be NULL (not computed).  grad_in is overwritten;
 * grad_weights is zeroed then accumulated with fp32 atomics across node
 * chunks (rounding order varies from run to run). */
e3conv_status e3conv_linear_backward(e3conv_plan_t plan, int channels_out, float scale,
                                     const float* weights, const float* in, int64_t num_nodes,
                                     const float* grad_out, float* grad_in, float* grad_weights,
                                     void* hip_stream);

/* Receiver CSR on the device: row_ptr[b] = first edge whose receiver is >= b,
 * for b = 0..num_nodes, from the receiver of each edge (device int32[num_edges],
 * non-decreasing).  One thread per node, binary search; asynchronous.  For a
 * SENDER plan pass the (non-decreasing) senders instead: the result is the
 * sender CSR. */
e3conv_status e3conv_csr_from_receivers(const int32_t* receivers_sorted, int64_t num_edges,
                                        int64_t num_nodes, int32_t* row_ptr, void* hip_stream);

/* Receiver processing order that improves cache reuse of the gathered sender
 * rows (host only; once per graph, like the CSR).  From the host CSR (row_ptr,
 * src) it grows breadth-first clusters of about `cluster` receivers over the
 * in-neighbour graph (seeds in index order) and writes their concatenation, a
 * permutation of 0..num_nodes-1, to the host array order[num_nodes].  The
 * graph is validated first (E3CONV_ERR_GRAPH on failure).  Pass the result,
 * copied to the device, as `order` to e3conv_forward / e3conv_backward. */
e3conv_status e3conv_receiver_order(const int32_t* row_ptr, const int32_t* src, int64_t num_nodes,
                                    int64_t num_edges, int cluster, int32_t* order);

/* Node relabeling for locality (host only; once per graph).  The convolution
 * commutes with renaming the nodes (the page's formula sums over the edges into
 * each receiver, whatever the node ids): relabeled inputs give the relabeled
 * output.  This call renames node v to its rank in the order
 * e3conv_receiver_order(cluster) gives, so that index order is that processing
 * order: consecutive receivers share senders and their rows of s, y and out
 * sit next to each other in memory.  Outputs (host, caller-owned):
 *   node_new[num_nodes]  new id of old node v (a permutation);
 *   edge_perm[num_edges] old index of the k-th edge of the relabeled graph,
 *                        whose edges are sorted by new receiver, then by new
 *                        sender, then by old index.
 * The relabeled graph is src'[k] = node_new[src[edge_perm[k]]], dst'[k] =
 * node_new[dst[edge_perm[k]]]; its edge rows are y[edge_perm[k]] and
 * s[edge_perm[k]]; node rows move as x'[node_new[v]] = x[v], and the output
 * comes back as out[v] = out'[node_new[v]].  Validates the graph first
 * (E3CONV_ERR_GRAPH); cluster > 0. */
e3conv_status e3conv_relabel_nodes(const int32_t* row_ptr, const int32_t* src, int64_t num_nodes,
                                   int64_t num_edges, int cluster, int32_t* node_new,
                                   int32_t* edge_perm);

/* Forward of pair-stored edge data: the function whose reverse pass is
 * e3conv_backward_pairs (e3j Convolution page, the note on SENDER ordering:
 * symmetric graph, y_ba = (-1)^l y_ab, s_ba = s_ab).  The messages are summed
 * over the directed receiver CSR (src, row_ptr, order, num_edges = 2 *
 * num_pairs, exactly as e3conv_forward), but each edge reads its y and s rows
 * from the pair arrays: row k = pair_of[e] if that is >= 0, else row ~k with
 * the odd-l blocks of y negated (the edge is the reverse of the stored one).
 * y (num_pairs, num_y) and s (num_pairs, num_paths, C) hold one row per pair;
 * pair_of is device int32[num_edges] in [-num_pairs, num_pairs) (out of range
 * is undefined behaviour), as e3conv_pair_layout writes it.  Every s row is
 * read twice (once per direction), so the bytes equal e3conv_forward's; the
 * edge data takes half the memory.  x and out as e3conv_forward (fp32).
 * RECEIVER plans; E3CONV_ERR_UNSUPPORTED for a layout without this kernel. */
e3conv_status e3conv_forward_pairs(e3conv_plan_t plan, const float* x, const float* y, const float* s,
                                   const int32_t* src, const int32_t* row_ptr,
                                   const int32_t* pair_of, const int32_t* order, int64_t num_nodes,
                                   int64_t num_edges, int64_t num_pairs, float* out,
                                   void* hip_stream);

/* Pair storage for e3conv_backward_pairs (host only, once per graph, like the
 * receiver order).  From the host receiver CSR (row_ptr, src) of a graph that
 * holds b -> a whenever it holds a -> b, once each, without self loops (the
 * radius graphs of the gate-points page are such graphs), it picks one
 * directed edge per undirected pair and orders the picks: receivers in the
 * order e3conv_receiver_order(cluster) gives, each pair stored as its edge
 * into the endpoint that comes first in that order, the stored edges of one
 * receiver consecutive.  Nearby receivers then follow each other, which keeps
 * the rows the pair pass gathers in cache.  Writes
 *   stored[num_edges / 2]  the directed edge of each stored pair (so the pair
 *                          arrays are y[stored], s[stored], src[stored] and the
 *                          receivers of those edges);
 *   pair_of[num_edges]     for every directed edge e, the position k of its pair
 *                          in stored if e is the stored edge, else ~k = -k - 1
 *                          (e is the stored edge's reverse); the directed rows
 *                          of s are s_pair[k], those of y are y_pair[k] and
 *                          P y_pair[k] (the map e3conv_forward_pairs takes).
 * E3CONV_ERR_GRAPH if the graph is invalid (as e3conv_validate_graph), not
 * symmetric, has a repeated edge, a self loop or an odd number of edges. */
e3conv_status e3conv_pair_layout(const int32_t* row_ptr, const int32_t* src, int64_t num_nodes,
                                 int64_t num_edges, int cluster, int32_t* stored,
                                 int32_t* pair_of);

/* Check a graph (the e3j Convolution page, __call__: indices lie in
 * [0, num_nodes); the fused kernels need edges sorted by receiver): row_ptr[0]
 * = 0, row_ptr non-decreasing and within [0, num_edges], row_ptr[num_nodes] =
 * num_edges, every src in [0, num_nodes).  on_device = 0: host pointers, checked
 * on the host.  on_device = 1: device pointers; a synchronous convenience that
 * allocates a small device result buffer, runs the check on the default stream,
 * waits for it and frees the buffer (use e3conv_validate_graph_async where
 * that is not wanted).  Returns E3CONV_OK, or E3CONV_ERR_GRAPH with the
 * first offending row_ptr index and/or edge in the detail. */
e3conv_status e3conv_validate_graph(const int32_t* src, const int32_t* row_ptr,
                                    int64_t num_nodes, int64_t num_edges, int on_device);

/* The device check of e3conv_validate_graph without allocation or
 * synchronisation: enqueued on hip_stream, it writes into the caller's device
 * buffer result (int32[4]): result[0] = number of violations (0: the graph is
 * valid), result[1] = first index i with row_ptr[i] outside [0, num_edges]
 * (or not 0 at i = 0, not num_edges at i = num_nodes) or with row_ptr[i + 1]
 * < row_ptr[i] (INT32_MAX if none), result[2] = first edge whose sender is out of range
 * (INT32_MAX if none), result[3] = 0.  The caller reads result after the
 * stream reaches it.  E3CONV_ERR_INVALID_ARGUMENT for NULL pointers or sizes
 * that do not fit int32 indices. */
e3conv_status e3conv_validate_graph_async(const int32_t* src, const int32_t* row_ptr,
                                          int64_t num_nodes, int64_t num_edges, int32_t* result,
                                          void* hip_stream);

/* e3conv_validate_graph(on_device = 1) for callers that cannot allocate
 * device memory (serving loops and harnesses that forbid hipMalloc): the same
 * check, status and detail, with the 4-int result held in a static device
 * array of the library (one per device, allocated with the code object and
 * kept until the process ends) instead of a per-call allocation.  The check
 * is enqueued on hip_stream, which the call then synchronises (it reads the
 * result back).  The array's size does not depend on the graph; sizes are
 * limited as for e3conv_validate_graph (int32 indices), else
 * E3CONV_ERR_INVALID_ARGUMENT.  Every call on one device shares that array:
 * calls that overlap on one device (from several threads or streams) race
 * and must be serialised by the caller. */
e3conv_status e3conv_validate_graph_noalloc(const int32_t* src, const int32_t* row_ptr,
                                            int64_t num_nodes, int64_t num_edges,
                                            void* hip_stream);

/* Streaming reference (measurement aid, not part of the convolution): copies
 * `bytes` from src to dst with 16-byte non-temporal loads and stores, or, with
 * dst = NULL, only reads src.  It measures the bandwidth this device attains
 * for plain streaming, the practical ceiling beside the published HBM peak,
 * and serves as the known-size kernel that scales memory counters.  bytes must
 * be a multiple of 16 and both buffers 16-byte aligned; asynchronous on
 * hip_stream.  src is never written. */
e3conv_status e3conv_stream_reference(const void* src, void* dst, size_t bytes, void* hip_stream);

/* Tuning: select a kernel variant for this plan (0 = default).  Variants
 * differ in how lanes map to channels and edges and compute the same result
 * to fp32 rounding, with one exception: for 64x(0e+1o+2e), SH lmax 3 ->
 * 64x(0e+1o+2e+3o) with bf16 operands, RECEIVER forward variants 6 and 7 run
 * the product on bf16 matrix instructions and round s x (and K, the edge's CG
 * matrix from y; variant 7 keeps K as two bf16 parts) to bf16, an error of at
 * most about 2^-7 of sum |C||y||s||x| per output element.  A variant index
 * beyond the list of an ordering or dtype selects its default.  Returns
 * E3CONV_ERR_UNSUPPORTED for a variant beyond every list.  Plans are
 * otherwise immutable; set variants before sharing a plan across threads. */
e3conv_status e3conv_plan_set_variant(e3conv_plan_t plan, int forward_variant, int backward_variant);

/* Number of forward / backward variants compiled for this plan's layout. */
e3conv_status e3conv_plan_num_variants(e3conv_plan_t plan, e3conv_dtype in_dtype,
                                       int* forward_variants, int* backward_variants);

const char* e3conv_status_string(e3conv_status status);
const char* e3conv_last_error_detail(void);   /* thread-local, never NULL */

#ifdef __cplusplus
}
#endif

#endif /* E3CONV_H */
