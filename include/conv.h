/*
 * conv.h -- C ABI of the 2-D convolution and its two derivatives, in the same
 * library as attn.h (whose status and element-type enums it uses).
 *
 * "Meganeura: Portable GPU Training and Inference through Vulkan and Metal"
 * (arXiv 2608.01563) treats convolution as a graph node with local input and
 * weight derivatives (Section 3.1), lowers them to implicit-GEMM kernels
 * (Section 3.3), and finds its weight-gradient and input-gradient kernels to
 * be most of a ResNet-50 training step (Section 7.3).  The operation is the
 * deep-learning cross-correlation with zero padding and a stride, NHWC:
 *   y[n,p,q,k]  = sum_{r,s,c} x[n, p*sh + r - ph, q*sw + s - pw, c] * w[k,r,s,c]
 *                 (x outside the image is zero)
 *   P = (H + 2*ph - R) / sh + 1,  Q = (W + 2*pw - S) / sw + 1  (rounded down)
 * and, for a loss whose gradient with respect to y is dy,
 *   dx[n,h,w,c] = sum over (p,q,r,s) with p*sh + r - ph = h and
 *                 q*sw + s - pw = w of sum_k dy[n,p,q,k] * w[k,r,s,c]
 *   dw[k,r,s,c] = sum_{n,p,q} dy[n,p,q,k] * x[n, p*sh + r - ph, q*sw + s - pw, c]
 *
 * Conventions (as attn.h unless stated):
 *  - x, dx [batch, height, width, channels]; w, dw [filters, kh, kw,
 *    channels]; y, dy [batch, P, Q, filters]; all contiguous row-major DEVICE
 *    pointers owned by the caller, aligned to the element size.  Outputs are
 *    overwritten (not accumulated); inputs are never written; outputs must
 *    not alias inputs.
 *  - dtype ATTN_F32: float32 tensors, f32 MFMA operands and accumulation
 *    (strict f32).  ATTN_BF16: bfloat16 tensors and MFMA operands, float32
 *    accumulation, outputs rounded to nearest-even bf16.  Other values:
 *    ATTN_ERR_UNSUPPORTED.
 *  - Sizes: every extent positive, strides positive, paddings non-negative,
 *    the padded image at least the filter size, and every tensor and GEMM
 *    extent below 2^31 elements; otherwise (or for a null or misaligned
 *    pointer) ATTN_ERR_INVALID_ARG, before anything is enqueued.
 *  - Calls enqueue on `stream` (a hipStream_t; NULL = the null stream) and
 *    return; results are valid once the stream is synchronised.  A launch
 *    failure returns ATTN_ERR_HIP.
 */
#ifndef CONV_MI355X_H
#define CONV_MI355X_H

#include <stddef.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* y from x and w (forward). */
attn_status_t conv2d_fwd(attn_dtype_t dtype, const void* x, const void* w, void* y, int batch,
                         int height, int width, int channels, int filters, int kh, int kw,
                         int stride_h, int stride_w, int pad_h, int pad_w, void* stream);

/* dx from dy and w (the input derivative). */
attn_status_t conv2d_bwd_data(attn_dtype_t dtype, const void* dy, const void* w, void* dx,
                              int batch, int height, int width, int channels, int filters,
                              int kh, int kw, int stride_h, int stride_w, int pad_h, int pad_w,
                              void* stream);

/*
 * dw from x and dy (the weight derivative).  Its reduction over
 * batch * P * Q is split into slices whose float32 partial sums go to a
 * caller-owned device workspace, [slices][filters][kh*kw*channels], and are
 * added in slice order (deterministic).  conv2d_bwd_filter_workspace_size
 * returns the bytes needed (0 when the shape takes one slice, or for an
 * invalid shape); a smaller, null or not 16-byte aligned workspace returns
 * ATTN_ERR_WORKSPACE.
 */
size_t conv2d_bwd_filter_workspace_size(attn_dtype_t dtype, int batch, int height, int width,
                                        int channels, int filters, int kh, int kw, int stride_h,
                                        int stride_w, int pad_h, int pad_w);
attn_status_t conv2d_bwd_filter(attn_dtype_t dtype, const void* x, const void* dy, void* dw,
                                void* workspace, size_t workspace_bytes, int batch, int height,
                                int width, int channels, int filters, int kh, int kw,
                                int stride_h, int stride_w, int pad_h, int pad_w, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONV_MI355X_H */
