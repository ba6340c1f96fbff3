// libselscan - the depthwise convolutions in front of the scan, for MI355X (gfx950), behind the
// C ABI declared in include/selscan.h.
//
// "Mamba Series from Selective State Spaces to Visual State Space Models", section 方法设计
// (architecture diagram): the Mamba block's scan branch is Linear -> Conv1D(k=4) -> SiLU ->
// SSM, the VSS block's is Linear -> DWConv 3x3 -> SiLU -> SS2D (section 关键代码,
// SS2Dv0.forwardv0: conv2d, then act).  The convolution's output also feeds the projections
// that make delta, B and C, so it is written to memory whatever the scan does; these kernels
// produce it in one pass over the input, at the bandwidth of the input and output streams.
//
// Work decomposition (both kernels): a thread owns 8 consecutive channels (one 16-byte vector
// of bf16, two of fp32) and a short run of positions; consecutive threads take consecutive
// channel groups of the same positions, so a wave's loads and stores are contiguous row
// segments.  A thread issues every load of its run at once, as raw io bits (converted to fp32
// where used), so each wave keeps many rows in flight: the kernels are bound by memory
// latency x parallelism otherwise, not by the stream bandwidth.
//  - causal_conv1d: a run of kR1 = 16 steps plus the K-1 rows before it (those come from the
//    caches: the previous run's thread read them).
//  - dwconv2d: R pixels of one image row (8 for bf16, 2 for fp32) and the 3 x (R + 2)
//    neighbourhood around them (rows above and below are neighbouring threads' rows: cache hits).
// The filters of a thread's 8 channels are contiguous ([dim][taps]) and read as 16-byte vectors.
#include "selscan_common.h"

namespace {

constexpr int kR1 = 16;  // steps per thread (conv1d)
template <typename T>
constexpr int rw_of() { return sizeof(T) == 2 ? 8 : 2; }  // pixels per thread along a row (dwconv2d)

struct Conv1dParams {
    const void *x;
    const float *w, *bias;  // [dim][K], [dim]
    const void *state_in;   // [batch][K-1][dim] io dtype, or NULL (zeros)
    void *state_out;        // [batch][K-1][dim] io dtype, or NULL
    void *out;
    int64_t L, dim;
    int batch, silu, vec, wvec, ncg, ntb;
};

template <typename T>
__device__ __forceinline__ void row8(const T *p, int nv, bool vec, float v[8]) {
    const Raw8<T> r = load_raw8(p, nv, vec);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = raw_f32(r, e);
}

__device__ __forceinline__ float act(float v, int silu_) { return silu_ ? silu(v) : v; }

// This thread's index in the logical order (channel group fastest, then position).  Workgroups
// are dealt round-robin over the 8 XCDs; the remap gives each XCD a contiguous range of logical
// workgroups, so the image rows a thread shares with its neighbours above and below are read on
// the same XCD, from its L2 (measured: 30.0 against 31.6 us on the VMamba stage-1 map).  The
// 1-D kernel keeps the plain order: the remap made it slower (565 against 539 us on the
// Mamba-1.4B-layer shape), its shared rows being only 3 in 19.
__device__ __forceinline__ int64_t logical_tid() {
    const int G = gridDim.x, bi = blockIdx.x, q8 = G >> 3;
    const int blk = bi < (q8 << 3) ? (bi & 7) * q8 + (bi >> 3) : bi;
    return (int64_t)blk * 256 + threadIdx.x;
}

// the TAPS filter taps of channels c0 .. c0+7 ([dim][TAPS] fp32), f[e * TAPS + i]; zeros past nv
template <int TAPS>
__device__ __forceinline__ void filters8(const float *w, int64_t c0, int nv, bool vec, float f[8 * TAPS]) {
    if (vec && nv == 8 && (8 * TAPS) % 4 == 0) {
        const float4 *q = (const float4 *)(w + c0 * TAPS);
#pragma unroll
        for (int k = 0; k < 2 * TAPS; ++k) {
            const float4 v = q[k];
            f[4 * k] = v.x, f[4 * k + 1] = v.y, f[4 * k + 2] = v.z, f[4 * k + 3] = v.w;
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 8 * TAPS; ++k) f[k] = k / TAPS < nv ? w[c0 * TAPS + k] : 0.f;
}

template <typename T, int K>
__global__ __launch_bounds__(256) void causal_conv1d_kernel(Conv1dParams p) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)p.batch * p.ntb * p.ncg) return;
    const int cg = (int)(gid % p.ncg);
    const int64_t rest = gid / p.ncg;
    const int tb = (int)(rest % p.ntb), b = (int)(rest / p.ntb);
    const int64_t c0 = (int64_t)cg * 8, L = p.L, dim = p.dim;
    const int nv = (int)(dim - c0 < 8 ? dim - c0 : 8);
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x + (int64_t)b * L * dim + c0;
    const T *st = p.state_in ? (const T *)p.state_in + (int64_t)b * (K - 1) * dim + c0 : nullptr;
    T *out = (T *)p.out + (int64_t)b * L * dim + c0;

    float f[8 * K], bs[8];
    filters8<K>(p.w, c0, nv, p.wvec != 0, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) bs[e] = p.bias && e < nv ? p.bias[c0 + e] : 0.f;
    const int64_t t0 = (int64_t)tb * kR1;
    // rows t0-(K-1) .. t0+kR1-1 of the sequence extended by the state rows in front (zero rows
    // without a state and past the end), all requested before any is used
    Raw8<T> raw[kR1 + K - 1];
#pragma unroll
    for (int i = 0; i < kR1 + K - 1; ++i) {
        const int64_t s = t0 - (K - 1) + i;
        raw[i] = Raw8<T>{};
        if (s >= 0 && s < L) raw[i] = load_raw8(x + s * dim, nv, vec);
        else if (s < 0 && st) raw[i] = load_raw8(st + (K - 1 + s) * dim, nv, vec);
    }
#pragma unroll
    for (int u = 0; u < kR1; ++u) {
        if (t0 + u >= L) break;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = bs[e];
#pragma unroll
            for (int i = 0; i < K; ++i) a = fmaf(f[e * K + i], raw_f32(raw[u + i], e), a);
            v[e] = act(a, p.silu);
        }
        store8(out + (t0 + u) * dim, nv, vec, v);
    }
    if (p.state_out && tb == p.ntb - 1) {
        // the last K-1 input rows (state rows where the sequence is shorter), raw copies
        T *so = (T *)p.state_out + (int64_t)b * (K - 1) * dim + c0;
#pragma unroll
        for (int r = 0; r < K - 1; ++r) {
            const int64_t s = L - (K - 1) + r;
            float v[8];
            if (s >= 0) row8(x + s * dim, nv, vec, v);
            else if (st) row8(st + (K - 1 + s) * dim, nv, vec, v);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            store8(so + r * dim, nv, vec, v);
        }
    }
}

struct Dw2dParams {
    const void *x;
    const float *w, *bias;  // [dim][3][3], [dim]
    void *out;
    int64_t dim;
    int H, W, batch, silu, vec, wvec, ncg, nwb;
};

template <typename T>
__global__ __launch_bounds__(256) void dwconv2d3_kernel(Dw2dParams p) {
    const int64_t gid = logical_tid();
    if (gid >= (int64_t)p.batch * p.H * p.nwb * p.ncg) return;
    const int cg = (int)(gid % p.ncg);
    int64_t rest = gid / p.ncg;
    const int wb = (int)(rest % p.nwb);
    rest /= p.nwb;
    const int h = (int)(rest % p.H), b = (int)(rest / p.H);
    const int64_t c0 = (int64_t)cg * 8, dim = p.dim;
    const int H = p.H, W = p.W;
    const int nv = (int)(dim - c0 < 8 ? dim - c0 : 8);
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x + (int64_t)b * H * W * dim + c0;
    T *out = (T *)p.out + (int64_t)b * H * W * dim + c0;

    constexpr int R = rw_of<T>();
    float f[72], bs[8];
    filters8<9>(p.w, c0, nv, p.wvec != 0, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) bs[e] = p.bias && e < nv ? p.bias[c0 + e] : 0.f;
    const int w0 = wb * R;
    // the 3 x (R+2) neighbourhood: rows h-1 .. h+1, columns w0-1 .. w0+R (zeros outside the map),
    // all requested before any is used
    Raw8<T> raw[3][R + 2];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int hh = h - 1 + i;
#pragma unroll
        for (int j = 0; j < R + 2; ++j) {
            const int c = w0 - 1 + j;
            raw[i][j] = Raw8<T>{};
            if (hh >= 0 && hh < H && c >= 0 && c < W) raw[i][j] = load_raw8(x + ((int64_t)hh * W + c) * dim, nv, vec);
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
        if (w0 + u >= W) break;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = bs[e];
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j) a = fmaf(f[e * 9 + i * 3 + j], raw_f32(raw[i][u + j], e), a);
            v[e] = act(a, p.silu);
        }
        store8(out + ((int64_t)h * W + w0 + u) * dim, nv, vec, v);
    }
}

int launch_grid(const void *kern, int64_t threads, void *args, void *stream) {
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    void *a[] = {args};
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)blocks), dim3(256), a, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        record_hip_error(e);
        return SELSCAN_E_HIP;
    }
    return SELSCAN_OK;
}

template <typename T>
int conv1d_launch(Conv1dParams &c, int K, void *stream) {
    const int64_t threads = (int64_t)c.batch * c.ntb * c.ncg;
    switch (K) {
        case 1: return launch_grid((const void *)&causal_conv1d_kernel<T, 1>, threads, &c, stream);
        case 2: return launch_grid((const void *)&causal_conv1d_kernel<T, 2>, threads, &c, stream);
        case 3: return launch_grid((const void *)&causal_conv1d_kernel<T, 3>, threads, &c, stream);
        default: return launch_grid((const void *)&causal_conv1d_kernel<T, 4>, threads, &c, stream);
    }
}

}  // namespace

extern "C" {

int causal_conv1d_fwd(const void *x, const float *weight, const float *bias, const void *state_in, void *state_out,
                      unsigned flags, void *out, int64_t batch, int64_t seqlen, int64_t dim, int64_t width,
                      int io_dtype, void *stream) {
    if (batch < 0 || seqlen < 0 || dim < 0 || width < 0) return SELSCAN_E_SHAPE;
    if (io_dtype != SELSCAN_F32 && io_dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (flags & ~SELSCAN_FLAG_SILU) return SELSCAN_E_UNSUPPORTED;
    if (width < 1 || width > 4) return SELSCAN_E_UNSUPPORTED;
    if (batch == 0 || dim == 0 || (seqlen == 0 && !state_out)) return SELSCAN_OK;
    if (!weight || (seqlen > 0 && (!x || !out))) return SELSCAN_E_NULL;
    const size_t s = io_dtype == SELSCAN_BF16 ? 2 : 4;
    const void *io[] = {x, state_in, state_out, out};
    for (const void *q : io)
        if (q && !aligned(q, s)) return SELSCAN_E_ALIGN;
    if (!aligned(weight, 4) || (bias && !aligned(bias, 4))) return SELSCAN_E_ALIGN;
    const size_t tok = (size_t)batch * seqlen * dim * s, sts = (size_t)batch * (width - 1) * dim * s;
    const Span in[] = {{x, tok}, {weight, (size_t)dim * width * 4}, {bias, (size_t)dim * 4}, {state_in, sts}};
    const Span outs[] = {{out, tok}, {state_out, sts}};
    for (const Span &o : outs)
        for (const Span &q : in)
            if (overlap(o, q)) return SELSCAN_E_ALIAS;
    if (overlap(outs[0], outs[1])) return SELSCAN_E_ALIAS;
    if (batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    Conv1dParams c;
    c.x = x, c.w = weight, c.bias = bias, c.state_in = state_in, c.state_out = state_out, c.out = out;
    c.L = seqlen, c.dim = dim, c.batch = (int)batch, c.silu = (flags & SELSCAN_FLAG_SILU) ? 1 : 0;
    const void *rows[] = {x, state_in, state_out, out};
    bool vec = dim % 8 == 0;
    for (const void *q : rows)
        if (q && !aligned(q, 16)) vec = false;
    c.vec = vec;
    c.wvec = aligned(weight, 16);
    c.ncg = (int)((dim + 7) / 8);
    const int64_t ntb = (seqlen + kR1 - 1) / kR1;
    if (ntb > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    c.ntb = ntb > 0 ? (int)ntb : 1;  // one (empty) run when only the state is copied
    if (io_dtype == SELSCAN_BF16) return conv1d_launch<uint16_t>(c, (int)width, stream);
    return conv1d_launch<float>(c, (int)width, stream);
}

int dwconv2d_fwd(const void *x, const float *weight, const float *bias, unsigned flags, void *out, int64_t batch,
                 int64_t H, int64_t W, int64_t dim, int64_t ksize, int io_dtype, void *stream) {
    if (batch < 0 || H < 0 || W < 0 || dim < 0 || ksize < 0) return SELSCAN_E_SHAPE;
    if (io_dtype != SELSCAN_F32 && io_dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (flags & ~SELSCAN_FLAG_SILU) return SELSCAN_E_UNSUPPORTED;
    if (ksize != 3) return SELSCAN_E_UNSUPPORTED;
    if (H > 0x7FFFFFFF || W > 0x7FFFFFFF || batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    if (batch == 0 || H == 0 || W == 0 || dim == 0) return SELSCAN_OK;
    if (!x || !weight || !out) return SELSCAN_E_NULL;
    const size_t s = io_dtype == SELSCAN_BF16 ? 2 : 4;
    if (!aligned(x, s) || !aligned(out, s)) return SELSCAN_E_ALIGN;
    if (!aligned(weight, 4) || (bias && !aligned(bias, 4))) return SELSCAN_E_ALIGN;
    const size_t tok = (size_t)batch * H * W * dim * s;
    const Span o{out, tok};
    if (overlap(o, {x, tok}) || overlap(o, {weight, (size_t)dim * 9 * 4}) || overlap(o, {bias, (size_t)dim * 4}))
        return SELSCAN_E_ALIAS;
    Dw2dParams c;
    c.x = x, c.w = weight, c.bias = bias, c.out = out, c.dim = dim;
    c.H = (int)H, c.W = (int)W, c.batch = (int)batch, c.silu = (flags & SELSCAN_FLAG_SILU) ? 1 : 0;
    c.vec = dim % 8 == 0 && aligned(x, 16) && aligned(out, 16);
    c.wvec = aligned(weight, 16);
    c.ncg = (int)((dim + 7) / 8);
    const int R = io_dtype == SELSCAN_BF16 ? rw_of<uint16_t>() : rw_of<float>();
    c.nwb = (int)((W + R - 1) / R);
    const int64_t threads = (int64_t)batch * H * c.nwb * c.ncg;
    if (io_dtype == SELSCAN_BF16) return launch_grid((const void *)&dwconv2d3_kernel<uint16_t>, threads, &c, stream);
    return launch_grid((const void *)&dwconv2d3_kernel<float>, threads, &c, stream);
}

}  // extern "C"
