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
        store8_stream(out + (t0 + u) * dim, nv, vec, v);
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

// ---- backward -------------------------------------------------------------------------------
// The chain rule through v = bias + sum of taps, out = act(v): dv = dout act'(v) (act' = 1 without
// the SiLU); every tap spreads dv back to the input it read (dx, and for the 1-D convolution the
// carried state rows), dw collects input x dv and dbias collects dv.  Three launches:
//  1. *_bwd_dv:  v recomputed from the input neighbourhood (as the forward kernels do), and each
//     thread's running sums of input x dv and dv over several runs written as one partial row
//     per thread group (no atomics); the 2-D kernel also writes dv to an fp32 workspace (dv
//     rounded to bf16 would add a second rounding to a bf16 dx);
//  2. *_bwd_dx:  dx as the transposed convolution of dv (the taps read in mirror order) -- the
//     1-D kernel recomputes the dv it needs from the inputs (a run of 8 steps needs K-1 more),
//     the 2-D kernel reads it back (a 3 x 3 neighbourhood of dv would need 5 x 5 inputs);
//  3. conv_bwd_reduce: dw and dbias as the sums of the partial rows, as a tree of fixed shape
//     (blocks of 64 rows x 64 columns, repeated until one row is left), so the results are the
//     same from run to run.

__device__ __forceinline__ float act_grad(float v, int silu_) {
    if (!silu_) return 1.f;
    const float s = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v * kLog2e));
    return s * (1.f + v * (1.f - s));
}

// 8 fp32 values of a row of the dv workspace (zeros past nv)
__device__ __forceinline__ void load_dv8(const float *p, int nv, bool vec, float v[8]) {
    if (vec && nv == 8) {
        const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < nv ? p[e] : 0.f;
}

__device__ __forceinline__ void store_dv8(float *p, int nv, bool vec, const float v[8]) {
    if (vec && nv == 8) {
        *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < nv) p[e] = v[e];
}

struct ConvBwdParams {
    const void *x, *dout, *state_in;
    const float *w, *bias;  // [dim][taps], [dim]
    float *dv;              // 2-D: [batch][H * W][dim] fp32
    float *part;            // [nparts][dim][taps + 1]: sums of input x dv per tap, then of dv
    void *dx, *dstate;      // dstate: [batch][K-1][dim] (1-D only), nullable
    float *dw, *dbias;
    int64_t L, dim;         // positions per batch row (1-D: seqlen; 2-D: H * W)
    int H, W, batch, silu, vec, wvec, ncg;
    int nrun;               // runs per batch row (1-D: steps / run; 2-D: row groups)
    int per;                // runs (1-D) or image rows (2-D) per thread in conv_bwd_dv
    int ngrp;               // thread groups per batch row in conv_bwd_dv (partial rows per batch row)
    int nwb;                // 2-D: pixel blocks per image row
    int nparts, taps;
};

// 1-D, launch 1: thread (b, group g, channel group); runs g*per .. g*per+per-1 of kRB steps
template <typename T, int K>
__global__ __launch_bounds__(256) void conv1d_bwd_dv(ConvBwdParams p) {
    constexpr int R = sizeof(T) == 2 ? 16 : 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)p.batch * p.ngrp * p.ncg) return;
    const int cg = (int)(gid % p.ncg);
    const int64_t rest = gid / p.ncg;
    const int grp = (int)(rest % p.ngrp), b = (int)(rest / p.ngrp);
    const int64_t c0 = (int64_t)cg * 8, L = p.L, dim = p.dim;
    const int nv = (int)(dim - c0 < 8 ? dim - c0 : 8);
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x + (int64_t)b * L * dim + c0;
    const T *dout = (const T *)p.dout + (int64_t)b * L * dim + c0;
    const T *st = p.state_in ? (const T *)p.state_in + (int64_t)b * (K - 1) * dim + c0 : nullptr;
    float f[8 * K], bs[8], sw[8 * K], sb[8];
    filters8<K>(p.w, c0, nv, p.wvec != 0, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bs[e] = p.bias && e < nv ? p.bias[c0 + e] : 0.f;
        sb[e] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8 * K; ++k) sw[k] = 0.f;
    for (int r = 0; r < p.per; ++r) {
        const int64_t t0 = ((int64_t)grp * p.per + r) * R;
        if (t0 >= L) break;
        Raw8<T> raw[R + K - 1], rd[R];
#pragma unroll
        for (int i = 0; i < R + K - 1; ++i) {
            const int64_t s = t0 - (K - 1) + i;
            raw[i] = Raw8<T>{};
            if (s >= 0 && s < L) raw[i] = load_raw8(x + s * dim, nv, vec);
            else if (s < 0 && st) raw[i] = load_raw8(st + (K - 1 + s) * dim, nv, vec);
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            rd[u] = Raw8<T>{};
            if (t0 + u < L) rd[u] = load_raw8(dout + (t0 + u) * dim, nv, vec);
        }
        // every step is guarded rather than the loop cut short: a constant trip count keeps the
        // unrolled arrays in registers
#pragma unroll
        for (int u = 0; u < R; ++u) {
            if (t0 + u < L) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float a = bs[e];
#pragma unroll
                    for (int i = 0; i < K; ++i) a = fmaf(f[e * K + i], raw_f32(raw[u + i], e), a);
                    const float g = raw_f32(rd[u], e) * act_grad(a, p.silu);
                    sb[e] += g;
#pragma unroll
                    for (int i = 0; i < K; ++i) sw[e * K + i] = fmaf(raw_f32(raw[u + i], e), g, sw[e * K + i]);
                }
            }
        }
    }
    float *pr = p.part + ((int64_t)b * p.ngrp + grp) * dim * (K + 1) + c0 * (K + 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (e >= nv) break;
#pragma unroll
        for (int i = 0; i < K; ++i) pr[e * (K + 1) + i] = sw[e * K + i];
        pr[e * (K + 1) + K] = sb[e];
    }
}

// 1-D, launch 2: thread (b, run, channel group); dx[s] = sum_i w[i] dv[s + K-1-i] for the run's
// 8 steps (and for the first run the K-1 state rows, s < 0), with dv[t] = dout[t] act'(v[t])
// recomputed for t = t0 .. t0+8+K-2 from the input rows t0-(K-1) .. t0+8+2K-3: the inputs are
// read again (mostly from the caches) instead of dv round-tripping through memory
template <typename T, int K>
__global__ __launch_bounds__(256) void conv1d_bwd_dx(ConvBwdParams p) {
    constexpr int R = 8, NT = R + K - 1, NX = R + 2 * K - 2;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)p.batch * p.nrun * p.ncg) return;
    const int cg = (int)(gid % p.ncg);
    const int64_t rest = gid / p.ncg;
    const int tb = (int)(rest % p.nrun), b = (int)(rest / p.nrun);
    const int64_t c0 = (int64_t)cg * 8, L = p.L, dim = p.dim;
    const int nv = (int)(dim - c0 < 8 ? dim - c0 : 8);
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x + (int64_t)b * L * dim + c0;
    const T *dout = (const T *)p.dout + (int64_t)b * L * dim + c0;
    const T *st = p.state_in ? (const T *)p.state_in + (int64_t)b * (K - 1) * dim + c0 : nullptr;
    T *dx = (T *)p.dx + (int64_t)b * L * dim + c0;
    float f[8 * K], bs[8];
    filters8<K>(p.w, c0, nv, p.wvec != 0, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) bs[e] = p.bias && e < nv ? p.bias[c0 + e] : 0.f;
    const int64_t t0 = (int64_t)tb * R;
    Raw8<T> raw[NX], rd[NT];  // input rows t0-(K-1) .. t0+NT-1, dout rows t0 .. t0+NT-1
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int64_t s = t0 - (K - 1) + i;
        raw[i] = Raw8<T>{};
        if (s >= 0 && s < L) raw[i] = load_raw8(x + s * dim, nv, vec);
        else if (s < 0 && st) raw[i] = load_raw8(st + (K - 1 + s) * dim, nv, vec);
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        rd[u] = Raw8<T>{};
        if (t0 + u < L) rd[u] = load_raw8(dout + (t0 + u) * dim, nv, vec);
    }
    // acc[j] collects dx of position t0 - (K-1) + j: the run's steps (j >= K-1) and, for the
    // first run, the state rows in front (j < K-1)
    float acc[NX][8];
#pragma unroll
    for (int j = 0; j < NX; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
    // guarded steps, constant trip counts: acc stays in registers
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        if (t0 + u < L) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = bs[e];
#pragma unroll
                for (int i = 0; i < K; ++i) a = fmaf(f[e * K + i], raw_f32(raw[u + i], e), a);
                const float g = raw_f32(rd[u], e) * act_grad(a, p.silu);
                // step t0+u read position t0+u-(K-1)+i through tap i
#pragma unroll
                for (int i = 0; i < K; ++i) acc[u + i][e] = fmaf(f[e * K + i], g, acc[u + i][e]);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (t0 + u < L) store8(dx + (t0 + u) * dim, nv, vec, acc[u + K - 1]);
    if (p.dstate && tb == 0) {
        T *ds = (T *)p.dstate + (int64_t)b * (K - 1) * dim + c0;
#pragma unroll
        for (int r = 0; r < K - 1; ++r) store8(ds + r * dim, nv, vec, acc[r]);
    }
}

// 2-D, launch 1: thread (b, row group, pixel block, channel group); rows grp*per .. +per-1,
// R pixels of each
// one wave per SIMD: the 9-tap filters and their running sums take 144 registers, and forcing
// two waves spills them (measured 0.31 against 0.22 ms for the whole backward on the VMamba map)
template <typename T>
__global__ __launch_bounds__(256) void dwconv2d3_bwd_dv(ConvBwdParams p) {
    constexpr int R = 2;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)p.batch * p.ngrp * p.nwb * p.ncg) return;
    const int cg = (int)(gid % p.ncg);
    int64_t rest = gid / p.ncg;
    const int wb = (int)(rest % p.nwb);
    rest /= p.nwb;
    const int grp = (int)(rest % p.ngrp), b = (int)(rest / p.ngrp);
    const int64_t c0 = (int64_t)cg * 8, dim = p.dim;
    const int H = p.H, W = p.W;
    const int nv = (int)(dim - c0 < 8 ? dim - c0 : 8);
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x + (int64_t)b * H * W * dim + c0;
    const T *dout = (const T *)p.dout + (int64_t)b * H * W * dim + c0;
    float *dv = p.dv + (int64_t)b * H * W * dim + c0;
    float f[72], bs[8], sw[72], sb[8];
    filters8<9>(p.w, c0, nv, p.wvec != 0, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bs[e] = p.bias && e < nv ? p.bias[c0 + e] : 0.f;
        sb[e] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 72; ++k) sw[k] = 0.f;
    const int w0 = wb * R;
    for (int r = 0; r < p.per; ++r) {
        const int h = grp * p.per + r;
        if (h >= H) break;
        Raw8<T> raw[3][R + 2], rd[R];
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
            rd[u] = Raw8<T>{};
            if (w0 + u < W) rd[u] = load_raw8(dout + ((int64_t)h * W + w0 + u) * dim, nv, vec);
        }
#pragma unroll
        for (int u = 0; u < R; ++u) {
            if (w0 + u >= W) break;
            float g[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = bs[e];
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int j = 0; j < 3; ++j) a = fmaf(f[e * 9 + i * 3 + j], raw_f32(raw[i][u + j], e), a);
                g[e] = raw_f32(rd[u], e) * act_grad(a, p.silu);
                sb[e] += g[e];
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int j = 0; j < 3; ++j)
                        sw[e * 9 + i * 3 + j] = fmaf(raw_f32(raw[i][u + j], e), g[e], sw[e * 9 + i * 3 + j]);
            }
            store_dv8(dv + ((int64_t)h * W + w0 + u) * dim, nv, vec, g);
        }
    }
    float *pr = p.part + (((int64_t)b * p.ngrp + grp) * p.nwb + wb) * dim * 10 + c0 * 10;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (e >= nv) break;
#pragma unroll
        for (int k = 0; k < 9; ++k) pr[e * 10 + k] = sw[e * 9 + k];
        pr[e * 10 + 9] = sb[e];
    }
}

// 2-D, launch 2: thread (b, image row, pixel block of 4, channel group); dx[h][w] =
// sum_{i,j} w[i][j] dv[h+1-i][w+1-j] (dv = 0 outside the map)
template <typename T>
__global__ __launch_bounds__(256) void dwconv2d3_bwd_dx(ConvBwdParams p) {
    constexpr int R = 4;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nwb = (p.W + R - 1) / R;
    if (gid >= (int64_t)p.batch * p.H * nwb * p.ncg) return;  // the launch covers batch x H x ceil(W/4) x ncg
    const int cg = (int)(gid % p.ncg);
    int64_t rest = gid / p.ncg;
    const int wb = (int)(rest % nwb);
    rest /= nwb;
    const int h = (int)(rest % p.H), b = (int)(rest / p.H);
    const int64_t c0 = (int64_t)cg * 8, dim = p.dim;
    const int H = p.H, W = p.W;
    const int nv = (int)(dim - c0 < 8 ? dim - c0 : 8);
    const bool vec = p.vec != 0;
    const float *dv = p.dv + (int64_t)b * H * W * dim + c0;
    T *dx = (T *)p.dx + (int64_t)b * H * W * dim + c0;
    float f[72];
    filters8<9>(p.w, c0, nv, p.wvec != 0, f);
    const int w0 = wb * R;
    float g[3][R + 2][8];  // dv rows h-1 .. h+1, columns w0-1 .. w0+R (zeros outside the map)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int hh = h - 1 + i;
#pragma unroll
        for (int j = 0; j < R + 2; ++j) {
            const int c = w0 - 1 + j;
            if (hh >= 0 && hh < H && c >= 0 && c < W) load_dv8(dv + ((int64_t)hh * W + c) * dim, nv, vec, g[i][j]);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) g[i][j][e] = 0.f;
        }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
        if (w0 + u >= W) break;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j) a = fmaf(f[e * 9 + i * 3 + j], g[2 - i][u + 2 - j][e], a);
            v[e] = a;
        }
        store8(dx + ((int64_t)h * W + w0 + u) * dim, nv, vec, v);
    }
}

struct ReduceParams {
    const float *src;  // [rows][cols]
    float *dst;        // [ceil(rows / 64)][cols], or NULL on the last level
    float *dw, *dbias; // the last level writes column d * (taps + 1) + k to dw[d][k] (k < taps) or dbias[d]
    int64_t rows, cols;
    int taps;
};

// launch 3, one level: block (column tile x, row tile y) adds rows 64 y .. 64 y + 63 of 64
// columns; thread (column c, slice s) adds rows 16 s .. 16 s + 15 of the tile in order, then the
// four slices are added in order
__global__ __launch_bounds__(256) void conv_bwd_reduce(ReduceParams p) {
    __shared__ float sm[4][64];
    const int c = threadIdx.x & 63, sl = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * 64 + c, t = blockIdx.y;
    float a = 0.f;
    if (col < p.cols) {
        const int64_t r0 = t * 64 + sl * 16;
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (r0 + k < p.rows) a += p.src[(r0 + k) * p.cols + col];
    }
    sm[sl][c] = a;
    __syncthreads();
    if (sl != 0 || col >= p.cols) return;
    const float v = ((sm[0][c] + sm[1][c]) + sm[2][c]) + sm[3][c];
    if (p.dst) {
        p.dst[t * p.cols + col] = v;
    } else {
        const int64_t d = col / (p.taps + 1);
        const int k = (int)(col % (p.taps + 1));
        if (k < p.taps) p.dw[d * p.taps + k] = v;
        else if (p.dbias) p.dbias[d] = v;
    }
}

// the tree: part -> t1 -> t2 -> t1 ... until a level has one row tile, which writes dw and dbias
int reduce_launch(const ConvBwdParams &c, float *t1, float *t2, void *stream) {
    ReduceParams r;
    r.src = c.part, r.dw = c.dw, r.dbias = c.dbias, r.rows = c.nparts, r.cols = c.dim * (c.taps + 1), r.taps = c.taps;
    float *bufs[2] = {t1, t2};
    for (int level = 0;; ++level) {
        const int64_t tiles = r.rows > 64 ? (r.rows + 63) / 64 : 1;
        r.dst = tiles > 1 ? bufs[level & 1] : nullptr;
        const int64_t bx = (r.cols + 63) / 64;
        if (bx > 0x7FFFFFFF || tiles > 65535) return SELSCAN_E_UNSUPPORTED;
        void *a[] = {&r};
        hipError_t e = hipLaunchKernel((const void *)&conv_bwd_reduce, dim3((unsigned)bx, (unsigned)tiles), dim3(256), a,
                                       0, (hipStream_t)stream);
        if (e != hipSuccess) {
            record_hip_error(e);
            return SELSCAN_E_HIP;
        }
        if (tiles == 1) return SELSCAN_OK;
        r.src = r.dst, r.rows = tiles;
    }
}

// the launch geometry of both backward convolutions, and the workspace it needs
struct ConvBwdPlan {
    int ngrp, per, nrun, nwb;
    int64_t parts;
    size_t dv_bytes, part_bytes, t1_bytes, t2_bytes;  // dv, partial rows, the reduction's two levels
    size_t total() const;
};

size_t up256(size_t v) { return (v + 255) / 256 * 256; }
size_t ConvBwdPlan::total() const { return up256(dv_bytes) + up256(part_bytes) + up256(t1_bytes) + up256(t2_bytes); }

void plan_tree(ConvBwdPlan &q, int64_t cols) {
    const int64_t r1 = (q.parts + 63) / 64, r2 = (r1 + 63) / 64;
    q.t1_bytes = (size_t)r1 * cols * 4;
    q.t2_bytes = (size_t)r2 * cols * 4;
}

// 1-D: runs of 16 (bf16) / 8 (fp32) steps for launch 1, 8 steps for launch 2; a launch-1 thread
// takes enough runs that there are about 2^17 of them (at most 16 runs each)
ConvBwdPlan plan_conv1d(int64_t batch, int64_t L, int64_t dim, int64_t K, int io_dtype) {
    ConvBwdPlan q{};
    const int64_t R1 = io_dtype == SELSCAN_BF16 ? 16 : 8, ncg = (dim + 7) / 8;
    const int64_t runs = (L + R1 - 1) / R1;
    int64_t per = (batch * runs * ncg + (1 << 17) - 1) >> 17;
    per = per < 1 ? 1 : (per > 16 ? 16 : per);
    q.per = (int)per;
    q.ngrp = (int)((runs + per - 1) / per);
    if (q.ngrp < 1) q.ngrp = 1;
    q.nrun = (int)((L + 7) / 8);
    if (q.nrun < 1) q.nrun = 1;  // one (empty) run still writes the state rows' gradient
    q.parts = batch * q.ngrp;
    q.dv_bytes = 0;  // launch 2 recomputes dv
    q.part_bytes = (size_t)q.parts * dim * (K + 1) * 4;
    plan_tree(q, dim * (K + 1));
    return q;
}

// 2-D: launch 1 takes 2 pixels of a row and a group of rows (8, or fewer rows per thread until
// there are 2^18 threads)
ConvBwdPlan plan_dwconv2d(int64_t batch, int64_t H, int64_t W, int64_t dim, int io_dtype) {
    ConvBwdPlan q{};
    const int64_t R = 2, ncg = (dim + 7) / 8;
    q.nwb = (int)((W + R - 1) / R);
    int64_t per = 8;
    while (per > 1 && batch * ((H + per - 1) / per) * q.nwb * ncg < (1 << 18)) per /= 2;
    q.per = (int)per;
    q.ngrp = (int)((H + per - 1) / per);
    q.parts = batch * q.ngrp * q.nwb;
    q.dv_bytes = (size_t)batch * H * W * dim * 4;
    q.part_bytes = (size_t)q.parts * dim * 10 * 4;
    plan_tree(q, dim * 10);
    return q;
}

template <typename T, int K>
int conv1d_bwd_launch(ConvBwdParams &c, float *t1, float *t2, void *stream) {
    int rc = launch_grid((const void *)&conv1d_bwd_dv<T, K>, (int64_t)c.batch * c.ngrp * c.ncg, &c, stream);
    if (rc == SELSCAN_OK)
        rc = launch_grid((const void *)&conv1d_bwd_dx<T, K>, (int64_t)c.batch * c.nrun * c.ncg, &c, stream);
    if (rc == SELSCAN_OK) rc = reduce_launch(c, t1, t2, stream);
    return rc;
}

template <typename T>
int conv1d_bwd_width(ConvBwdParams &c, int K, float *t1, float *t2, void *stream) {
    switch (K) {
        case 1: return conv1d_bwd_launch<T, 1>(c, t1, t2, stream);
        case 2: return conv1d_bwd_launch<T, 2>(c, t1, t2, stream);
        case 3: return conv1d_bwd_launch<T, 3>(c, t1, t2, stream);
        default: return conv1d_bwd_launch<T, 4>(c, t1, t2, stream);
    }
}

template <typename T>
int dwconv2d_bwd_launch(ConvBwdParams &c, float *t1, float *t2, void *stream) {
    int rc = launch_grid((const void *)&dwconv2d3_bwd_dv<T>, (int64_t)c.batch * c.ngrp * c.nwb * c.ncg, &c, stream);
    if (rc == SELSCAN_OK)
        rc = launch_grid((const void *)&dwconv2d3_bwd_dx<T>, (int64_t)c.batch * c.H * ((c.W + 3) / 4) * c.ncg, &c,
                         stream);
    if (rc == SELSCAN_OK) rc = reduce_launch(c, t1, t2, stream);
    return rc;
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

size_t causal_conv1d_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t width, int io_dtype) {
    if (batch <= 0 || seqlen < 0 || dim <= 0 || width < 1 || width > 4) return 0;
    return plan_conv1d(batch, seqlen, dim, width, io_dtype).total();
}

int causal_conv1d_bwd(const void *x, const float *weight, const float *bias, const void *state_in, const void *dout,
                      unsigned flags, void *dx, float *dweight, float *dbias, void *dstate_in, int64_t batch,
                      int64_t seqlen, int64_t dim, int64_t width, int io_dtype, void *workspace,
                      size_t workspace_bytes, void *stream) {
    if (batch < 0 || seqlen < 0 || dim < 0 || width < 0) return SELSCAN_E_SHAPE;
    if (io_dtype != SELSCAN_F32 && io_dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (flags & ~SELSCAN_FLAG_SILU) return SELSCAN_E_UNSUPPORTED;
    if (width < 1 || width > 4) return SELSCAN_E_UNSUPPORTED;
    if (batch > 0x7FFFFFFF || seqlen > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    if (batch == 0 || dim == 0) return SELSCAN_OK;
    if (!weight || !dweight || (seqlen > 0 && (!x || !dout || !dx))) return SELSCAN_E_NULL;
    const size_t s = io_dtype == SELSCAN_BF16 ? 2 : 4;
    const void *io[] = {x, state_in, dout, dx, dstate_in};
    for (const void *q : io)
        if (q && !aligned(q, s)) return SELSCAN_E_ALIGN;
    const void *f32[] = {weight, bias, dweight, dbias, workspace};
    for (const void *q : f32)
        if (q && !aligned(q, 4)) return SELSCAN_E_ALIGN;
    const size_t need = causal_conv1d_bwd_workspace_bytes(batch, seqlen, dim, width, io_dtype);
    if (!workspace || workspace_bytes < need) return SELSCAN_E_WORKSPACE;
    const size_t tok = (size_t)batch * seqlen * dim * s, sts = (size_t)batch * (width - 1) * dim * s;
    const size_t wb = (size_t)dim * width * 4, vb = (size_t)dim * 4;
    const Span in[] = {{x, tok}, {weight, wb}, {bias, vb}, {state_in, sts}, {dout, tok}};
    const Span out[] = {{dx, tok}, {dweight, wb}, {dbias, vb}, {dstate_in, sts}, {workspace, need}};
    constexpr int NO = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < NO; ++i) {
        for (const Span &q : in)
            if (overlap(out[i], q)) return SELSCAN_E_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(out[i], out[j])) return SELSCAN_E_ALIAS;
    }
    const ConvBwdPlan q = plan_conv1d(batch, seqlen, dim, width, io_dtype);
    ConvBwdParams c{};
    c.x = x, c.dout = dout, c.state_in = state_in, c.w = weight, c.bias = bias;
    c.dv = nullptr;
    c.part = (float *)((char *)workspace + up256(q.dv_bytes));
    c.dx = dx, c.dstate = width > 1 ? dstate_in : nullptr, c.dw = dweight, c.dbias = dbias;
    c.L = seqlen, c.dim = dim, c.batch = (int)batch, c.silu = (flags & SELSCAN_FLAG_SILU) ? 1 : 0;
    const void *rows[] = {x, state_in, dout, dx, dstate_in, workspace};
    bool vec = dim % 8 == 0;
    for (const void *r : rows)
        if (r && !aligned(r, 16)) vec = false;
    c.vec = vec;
    c.wvec = aligned(weight, 16);
    c.ncg = (int)((dim + 7) / 8);
    c.nrun = q.nrun, c.per = q.per, c.ngrp = q.ngrp;
    if (q.parts > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    c.nparts = (int)q.parts, c.taps = (int)width;
    float *t1 = (float *)((char *)c.part + up256(q.part_bytes));
    float *t2 = (float *)((char *)t1 + up256(q.t1_bytes));
    if (io_dtype == SELSCAN_BF16) return conv1d_bwd_width<uint16_t>(c, (int)width, t1, t2, stream);
    return conv1d_bwd_width<float>(c, (int)width, t1, t2, stream);
}

size_t dwconv2d_bwd_workspace_bytes(int64_t batch, int64_t H, int64_t W, int64_t dim, int io_dtype) {
    if (batch <= 0 || H <= 0 || W <= 0 || dim <= 0) return 0;
    return plan_dwconv2d(batch, H, W, dim, io_dtype).total();
}

int dwconv2d_bwd(const void *x, const float *weight, const float *bias, const void *dout, unsigned flags, void *dx,
                 float *dweight, float *dbias, int64_t batch, int64_t H, int64_t W, int64_t dim, int64_t ksize,
                 int io_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (batch < 0 || H < 0 || W < 0 || dim < 0 || ksize < 0) return SELSCAN_E_SHAPE;
    if (io_dtype != SELSCAN_F32 && io_dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (flags & ~SELSCAN_FLAG_SILU) return SELSCAN_E_UNSUPPORTED;
    if (ksize != 3) return SELSCAN_E_UNSUPPORTED;
    if (H > 0x7FFFFFFF || W > 0x7FFFFFFF || batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    if (dim == 0) return SELSCAN_OK;
    if (!weight || !dweight) return SELSCAN_E_NULL;
    const bool empty = batch == 0 || H == 0 || W == 0;
    if (!empty && (!x || !dout || !dx)) return SELSCAN_E_NULL;
    const size_t s = io_dtype == SELSCAN_BF16 ? 2 : 4;
    const void *io[] = {x, dout, dx};
    for (const void *q : io)
        if (q && !aligned(q, s)) return SELSCAN_E_ALIGN;
    const void *f32[] = {weight, bias, dweight, dbias, workspace};
    for (const void *q : f32)
        if (q && !aligned(q, 4)) return SELSCAN_E_ALIGN;
    const size_t need = empty ? 0 : dwconv2d_bwd_workspace_bytes(batch, H, W, dim, io_dtype);
    if (!empty && (!workspace || workspace_bytes < need)) return SELSCAN_E_WORKSPACE;
    const size_t tok = empty ? 0 : (size_t)batch * H * W * dim * s, wb = (size_t)dim * 9 * 4, vb = (size_t)dim * 4;
    const Span in[] = {{x, tok}, {weight, wb}, {bias, vb}, {dout, tok}};
    const Span out[] = {{dx, tok}, {dweight, wb}, {dbias, vb}, {workspace, need}};
    constexpr int NO = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < NO; ++i) {
        for (const Span &q : in)
            if (overlap(out[i], q)) return SELSCAN_E_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(out[i], out[j])) return SELSCAN_E_ALIAS;
    }
    ConvBwdParams c{};
    c.w = weight, c.bias = bias, c.dw = dweight, c.dbias = dbias, c.dim = dim, c.taps = 9;
    if (empty) {  // no pixels: dw and dbias are zero sums
        c.nparts = 0;
        return reduce_launch(c, nullptr, nullptr, stream);
    }
    const ConvBwdPlan q = plan_dwconv2d(batch, H, W, dim, io_dtype);
    c.x = x, c.dout = dout, c.dx = dx;
    c.dv = (float *)workspace;
    c.part = (float *)((char *)workspace + up256(q.dv_bytes));
    c.H = (int)H, c.W = (int)W, c.batch = (int)batch, c.silu = (flags & SELSCAN_FLAG_SILU) ? 1 : 0;
    c.vec = dim % 8 == 0 && aligned(x, 16) && aligned(dout, 16) && aligned(dx, 16) && aligned(workspace, 16);
    c.wvec = aligned(weight, 16);
    c.ncg = (int)((dim + 7) / 8);
    c.per = q.per, c.ngrp = q.ngrp, c.nwb = q.nwb;
    if (q.parts > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    c.nparts = (int)q.parts;
    float *t1 = (float *)((char *)c.part + up256(q.part_bytes));
    float *t2 = (float *)((char *)t1 + up256(q.t1_bytes));
    if (io_dtype == SELSCAN_BF16) return dwconv2d_bwd_launch<uint16_t>(c, t1, t2, stream);
    return dwconv2d_bwd_launch<float>(c, t1, t2, stream);
}

}  // extern "C"
