// selscan_common.h - what the forward and backward kernels of libselscan share: the tile
// geometry, the scan orders (visit), io conversions and row moves, fast division, host-side
// argument helpers.  Included by selscan_fwd.hip and selscan_bwd.hip only.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "selscan.h"

namespace selscan_rt {
// text of the calling thread's most recent rejected launch (selscan_last_hip_error)
extern thread_local char g_last_hip_error[160];
}  // namespace selscan_rt

namespace {

using selscan_rt::g_last_hip_error;

constexpr int kN = 16;                 // d_state supported by this version
constexpr int kK = 16;                 // consecutive scan steps per lane
constexpr int kLPR = 16;               // lanes per channel: one 16-lane DPP row, 4 channels per wave
constexpr int kCH = kLPR * kK;         // scan steps per chunk (256)
constexpr int kFP = kCH + 4;           // fp32 LDS pitch (floats) of the B, C and y tiles
constexpr int kTC = 16;                // channels per workgroup tile: 4 waves x 4 channels
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------------------------
// host-side helpers (pure host code: run before any HIP call)
// ------------------------------------------------------------------------------------

struct Span {
    const void *p;
    size_t bytes;
};

bool overlap(const Span &a, const Span &b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes, b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
    return a0 < b1 && b0 < a1;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

__host__ __device__ inline int64_t chunks_of(int64_t L) { return (L + kCH - 1) / kCH; }
size_t ckpt_bytes_for(int64_t batch, int64_t L, int64_t dim) {
    return (size_t)batch * (size_t)chunks_of(L) * (size_t)dim * kN * sizeof(float);
}

void record_hip_error(hipError_t e) {
    strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
}

// scan directions of an op (0: not an op)
int ndir_of(int op) {
    switch (op) {
        case SELSCAN_OP_FWD: return 1;
        case SELSCAN_OP_BIDIR: return 2;
        case SELSCAN_OP_SS2D:
        case SELSCAN_OP_LOCAL_SS2D: return 4;
        default: return 0;
    }
}

// Several directions run one after another in each workgroup, with the running sums in one
// fp32 workspace row set -- unless that leaves the chip short of workgroups (fewer than
// kSplitBelow channel tiles x batch rows, under two rounds of two per compute unit), in which
// case each workgroup takes one direction and writes its own partial rows, and a merge kernel
// adds them in direction order (the sums the sequential walk forms, in its order: fp32 addition
// is commutative, so the results are bit-identical).  Used when the caller's workspace holds
// the per-direction rows (the size queries ask for them in that case).
constexpr int64_t kSplitBelow = 1024;

inline bool split_wanted(int op, int64_t batch, int64_t dim) {
    return op != SELSCAN_OP_FWD && batch * ((dim + kTC - 1) / kTC) < kSplitBelow;
}

// sequence length and direction count of an op; H and W apply to the two-dimensional orders,
// whose seqlen must be H * W
int resolve_op(int op, int64_t seqlen, int64_t H, int64_t W, int64_t *L, int *ndir) {
    *ndir = ndir_of(op);
    if (*ndir == 0) return SELSCAN_E_UNSUPPORTED;
    *L = seqlen;
    if (op == SELSCAN_OP_SS2D || op == SELSCAN_OP_LOCAL_SS2D) {
        if (seqlen < 0 || H < 0 || W < 0) return SELSCAN_E_SHAPE;
        if (W > 0 && H > INT64_MAX / W) return SELSCAN_E_UNSUPPORTED;
        if (seqlen != H * W) return SELSCAN_E_SHAPE;
    }
    return SELSCAN_OK;
}

// n / d for 0 <= n < 2^31 as a multiply-high and a shift (Granlund-Montgomery): with
// 2^(s-1) < d <= 2^s, m = ceil(2^(31+s) / d) < 2^32 and floor(n m / 2^(31+s)) = floor(n / d).
struct FastDiv {
    uint32_t d, m, sh;
};
FastDiv make_div(uint32_t d) {
    FastDiv f{d, 0u, 0u};
    if (d <= 1) return f;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.m = (uint32_t)(((1ull << (31 + s)) + d - 1) / d);
    f.sh = s - 1;
    return f;
}
// (F: a FastDiv in any address space)
template <class F>
__device__ __forceinline__ uint32_t fdiv(uint32_t n, F &f) {
    return f.d <= 1 ? n : __umulhi(n, f.m) >> f.sh;
}

// the scan-order fields of a kernel's parameters (visit() reads them)
template <class P>
void set_order(P &a, int kind, int64_t L, int64_t H, int64_t W, int64_t win) {
    a.L = L, a.H = (int)H, a.Wd = (int)W, a.win = (int)win;
    a.dH = make_div((uint32_t)H);
    if (kind == SELSCAN_OP_LOCAL_SS2D) {
        a.dWin = make_div((uint32_t)win);
        a.dWin2 = make_div((uint32_t)(win * win));
        a.dNx = make_div((uint32_t)(W / win));
        a.dNy = make_div((uint32_t)(H / win));
    } else {
        a.dWin = a.dWin2 = a.dNx = a.dNy = make_div(1);
    }
}

// ------------------------------------------------------------------------------------
// device helpers
// ------------------------------------------------------------------------------------

template <typename T>
struct Io;
template <>
struct Io<float> {
    __device__ static float f32(float v) { return v; }
    __device__ static float to(float v) { return v; }
};
template <>
struct Io<uint16_t> {
    __device__ static float f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
    // round to nearest even (v_cvt_pk_bf16_f32); a NaN stays a NaN
    __device__ static uint16_t to(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
    __device__ static uint32_t to2(float lo, float hi) {
        typedef float f2 __attribute__((ext_vector_type(2)));
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const b2 r = __builtin_convertvector((f2){lo, hi}, b2);
        return __builtin_bit_cast(uint32_t, r);
    }
};

// position of chunk step s in an fp32 tile row (pieces of 4 floats)
__host__ __device__ constexpr int fpos(int s) { return ((s & 15) >> 2) * (kLPR * 4) + ((s >> 4) << 2) + (s & 3); }

template <bool V>
struct BoolC {
    static constexpr bool value = V;
};

// row (token or pixel) visited at scan step l, 0 <= l < L, by direction k; P carries L, H, Wd,
// win and the divisions by H, w, w*w, W/w, H/w
template <int KIND, typename P>
__device__ __forceinline__ int64_t visit(const P &p, int k, int64_t l) {
    const int64_t L = p.L;
    if constexpr (KIND == SELSCAN_OP_FWD) {
        return l;
    } else if constexpr (KIND == SELSCAN_OP_BIDIR) {
        return k == 0 ? l : L - 1 - l;
    } else if constexpr (KIND == SELSCAN_OP_SS2D) {
        // k = 0 row-major, 1 column-major, 2 and 3 the same orders reversed (L < 2^31)
        if (k >= 2) l = L - 1 - l;
        if ((k & 1) == 0) return l;
        const uint32_t u = (uint32_t)l, q = fdiv(u, p.dH), r = u - q * (uint32_t)p.H;
        return (int64_t)r * p.Wd + q;
    } else {
        // windowed: square windows of side w; k = 0 windows and their pixels row-major, 1 the
        // same on the transposed map, 2 and 3 reversed
        if (k >= 2) l = L - 1 - l;
        const uint32_t w = (uint32_t)p.win, u = (uint32_t)l;
        const uint32_t wi = fdiv(u, p.dWin2), r = u - wi * (w * w);
        const uint32_t ry = fdiv(r, p.dWin), rx = r - ry * w;
        if ((k & 1) == 0) {
            const uint32_t nx = (uint32_t)p.Wd / w, wy = fdiv(wi, p.dNx), wx = wi - wy * nx;
            return (int64_t)(wy * w + ry) * p.Wd + (wx * w + rx);
        }
        const uint32_t ny = (uint32_t)p.H / w, wy = fdiv(wi, p.dNy), wx = wi - wy * ny;
        // on the transposed map, row wy*w+ry is column wy*w+ry of this map and column wx*w+rx is a row
        return (int64_t)(wx * w + rx) * p.Wd + (wy * w + ry);
    }
}

// The kernel's arguments (a P, the kernel's only parameter), read afresh from the argument
// segment wherever this is called: the compiler keeps loaded arguments alive across the whole
// kernel and spills them into vector lanes, while a read through an opaque segment pointer is
// one scalar load at the use.
template <class P>
__device__ __forceinline__ const __attribute__((address_space(4))) P &fresh_args() {
    using CP = const __attribute__((address_space(4))) P;
    CP *pq = (CP *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(pq));
    return *pq;
}

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations only.  A
// __syncthreads would also wait for every global load and store the wave has in flight (its
// release fence drains vmcnt), which stalls on stores issued just before the barrier and on
// loads issued for the next chunk.  Within one scan direction no wave reads back global memory
// another wave of the workgroup wrote, so LDS ordering is all these barriers have to give; the
// barrier between directions (where the partial sums change hands) stays a full one.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Per-wave shader-clock cycles spent in each phase of a kernel's chunk loop, summed over the
// chunks: phase i's time runs from the previous add() (or mark()) to add(i).  Compiled in only
// for the diagnostic library (SELSCAN_PHASE_CLOCKS, libselscan_phases.so), which writes them,
// with the whole kernel's cycles, to a per-kernel record; otherwise every call is empty.
#ifdef SELSCAN_PHASE_CLOCKS
constexpr int kPhaseWaves = 1 << 14;  // waves the record holds: 8 u64 each
struct PhaseClock {
    unsigned long long acc[6] = {0, 0, 0, 0, 0, 0}, t = 0, t0 = __builtin_amdgcn_s_memtime();
    __device__ void mark() { t = __builtin_amdgcn_s_memtime(); }
    __device__ void add(int i) {
        const unsigned long long n = __builtin_amdgcn_s_memtime();
        acc[i] += n - t;
        t = n;
    }
    // lane 0 of the wave writes phases 0-5, the whole kernel, and 1 (written)
    __device__ void finish(unsigned long long *rec, int wave_id, int lane) {
        const unsigned long long end = __builtin_amdgcn_s_memtime();
        if (lane == 0 && wave_id < kPhaseWaves) {
#pragma unroll
            for (int i = 0; i < 6; ++i) rec[wave_id * 8 + i] = acc[i];
            rec[wave_id * 8 + 6] = end - t0;
            rec[wave_id * 8 + 7] = 1;
        }
    }
};
#else
struct PhaseClock {
    __device__ void mark() {}
    __device__ void add(int) {}
};
#endif

// softplus(w) = log(1 + e^w) = max(w, 0) + log1p(t), t = e^-|w|, on v_exp_f32 and v_log_f32.
// log1p(t) is taken as ln(u) t / (u - 1) with u = 1 + t rounded to fp32 (Kahan's form: the
// rounding error of u cancels between the logarithm and the denominator), and as t itself once
// u rounds to 1 (t below half an ulp of 1, where log1p(t) = t to fp32 precision).
__device__ __forceinline__ float softplus(float w) {
    const float t = __builtin_amdgcn_exp2f(-fabsf(w) * kLog2e);
    const float u = 1.f + t, d = u - 1.f;
    const float l = d == 0.f ? t : __builtin_amdgcn_logf(u) * kLn2 * (t * __builtin_amdgcn_rcpf(d));
    return fmaxf(w, 0.f) + l;
}

// Zero-order-hold input factor: Bbar x = (e^y - 1) / A * B x = delta phi(y) B x, with y = delta A,
// e = e^y and phi(y) = (e^y - 1) / y.  e - 1 from the exp carries its absolute rounding error
// (about 1e-7), which is a large relative error when |y| is small; there phi comes from its
// series, 1 + y/2 + y^2/6 + y^3/24 + y^4/120 (truncation below 5e-8 for |y| < 1/8), and
// elsewhere from (e - 1) / y (relative error about 1e-6 for |y| >= 1/8).  t = y log2(e), the
// exponent the recurrence's exp2 already takes.
__device__ __forceinline__ float zoh_phi(float e, float t) {
    const float y = t * kLn2;
    const float series = fmaf(y, fmaf(y, fmaf(y, fmaf(y, 1.f / 120.f, 1.f / 24.f), 1.f / 6.f), 0.5f), 1.f);
    const float direct = (e - 1.f) * __builtin_amdgcn_rcpf(y);
    return fabsf(y) < 0.125f ? series : direct;
}

// Its derivative, which the zero-order-hold gradient of A needs (d Bbar / dA = delta^2 phi'(y)):
// phi'(y) = (e^y (y - 1) + 1) / y^2 = (e^y - phi(y)) / y.  From the series 1/2 + y/3 + y^2/8 +
// y^3/30 + y^4/144 when |y| < 1/8 (truncation below 1e-7), else from (e - phi) / y (relative
// error below 2e-5 for |y| >= 1/8, falling as |y| grows); phi as zoh_phi gives it.
__device__ __forceinline__ float zoh_dphi(float e, float t, float phi) {
    const float y = t * kLn2;
    const float series =
        fmaf(y, fmaf(y, fmaf(y, fmaf(y, 1.f / 144.f, 1.f / 30.f), 1.f / 8.f), 1.f / 3.f), 0.5f);
    const float direct = (e - phi) * __builtin_amdgcn_rcpf(y);
    return fabsf(y) < 0.125f ? series : direct;
}

// silu(z) = z * sigmoid(z) on v_exp_f32 and v_rcp_f32 (large |z| saturates to 0 or z)
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// 8 consecutive io elements of one row as raw bits (bf16: 4 dwords; fp32: 8); elements past
// `n` read as 0
template <typename T>
struct Raw8 {
    uint32_t w[sizeof(T) * 2];
};

template <typename T>
__device__ __forceinline__ Raw8<T> load_raw8(const T *p, int n, bool vec) {
    Raw8<T> r;
    if (vec && n >= 8) {
        const uint4 q = *(const uint4 *)p;
        r.w[0] = q.x, r.w[1] = q.y, r.w[2] = q.z, r.w[3] = q.w;
        if constexpr (sizeof(T) == 4) {
            const uint4 q2 = *(const uint4 *)(p + 4);
            r.w[4] = q2.x, r.w[5] = q2.y, r.w[6] = q2.z, r.w[7] = q2.w;
        }
        return r;
    }
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 8; ++e) r.w[e] = e < n ? __float_as_uint(p[e]) : 0u;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = 2 * e < n ? (uint32_t)p[2 * e] : 0u;
            const uint32_t hi = 2 * e + 1 < n ? (uint32_t)p[2 * e + 1] : 0u;
            r.w[e] = lo | (hi << 16);
        }
    }
    return r;
}

// element e of a Raw8 as fp32 / as its raw io bits
template <typename T>
__device__ __forceinline__ float raw_f32(const Raw8<T> &r, int e) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(r.w[e]);
    else return __uint_as_float((e & 1) ? (r.w[e >> 1] & 0xFFFF0000u) : (r.w[e >> 1] << 16));
}

template <typename T>
__device__ __forceinline__ void store8(T *p, int n, bool vec, const float v[8]) {
    if (vec && n >= 8) {
        if constexpr (sizeof(T) == 4) {
            *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
            *(float4 *)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            *(uint4 *)p = make_uint4(Io<T>::to2(v[0], v[1]), Io<T>::to2(v[2], v[3]), Io<T>::to2(v[4], v[5]),
                                     Io<T>::to2(v[6], v[7]));
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < n) p[e] = Io<T>::to(v[e]);
}

// store8 with the streaming (nontemporal) hint on the vector path, for outputs that consecutive
// lanes write as whole cache lines and that the kernel does not read back.  (Outputs written as
// pieces of lines that other lanes or workgroups complete later keep the plain store: those
// pieces are merged in L2 before they go to memory.)
template <typename T>
__device__ __forceinline__ void store8_stream(T *p, int n, bool vec, const float v[8]) {
    if (vec && n >= 8) {
        if constexpr (sizeof(T) == 4) {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
            __builtin_nontemporal_store(a, (f32x4 *)p);
            __builtin_nontemporal_store(b, (f32x4 *)(p + 4));
        } else {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 q = {Io<T>::to2(v[0], v[1]), Io<T>::to2(v[2], v[3]), Io<T>::to2(v[4], v[5]),
                             Io<T>::to2(v[6], v[7])};
            __builtin_nontemporal_store(q, (u32x4 *)p);
        }
        return;
    }
    store8(p, n, vec, v);
}

__device__ __forceinline__ void load_f8(const float *p, int n, bool vec, float v[8]) {
    if (vec && n >= 8) {
        const float4 q = *(const float4 *)p, q2 = *(const float4 *)(p + 4);
        v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w, v[4] = q2.x, v[5] = q2.y, v[6] = q2.z, v[7] = q2.w;
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < n ? p[e] : 0.f;
}

}  // namespace
