// libselscan - selective state-space scan kernels for MI355X (gfx950) behind the C ABI
// declared in include/selscan.h.
//
// Method: "Mamba Series from Selective State Spaces to Visual State Space Models",
// section 选择性 SSM 的数学形式 (Abar = exp(delta A), selection of delta, B, C), insight 1
// (scan evaluated on chip with a parallel prefix scan, Abar/Bbar never written to HBM) and
// section 关键代码 (scan call with Ds, delta_bias, delta_softplus; the SS2D scan orders
// and merge; the SiLU gate); "从LSTM到Mamba" §2.1 (D skip) and §3.1 (bidirectional scan).
//
// Work decomposition (one kernel for every entry point):
//  - A workgroup owns one batch row and a tile of kCT = 16 channels, and walks every scan
//    direction of that tile over the whole sequence in chunks of kCH = 256 scan steps.
//  - A wave holds 4 channels, one per 16-lane DPP row.  Lane l of a row owns kK = 16
//    consecutive scan steps of its channel.  All fp32 state stays in VGPRs.
//  - Per chunk: x, delta (io dtype) are staged in LDS column-major per channel; B, C are
//    staged once as fp32 [state][step] and shared by the 16 channels of the tile.
//  - For each state n: pass 1 runs each lane's 16 steps from a zero state and keeps
//    dA = exp2(delta * A * log2 e) and u = delta * B * x in registers; the lanes' affine
//    maps (a, b) with a = exp2(A log2e * sum(delta)) are combined by a 4-step inclusive
//    Hillis-Steele scan across the 16-lane row (DPP row_shr, identity (1, 0)), with the
//    carry of the previous chunk folded into lane 0; pass 2 re-runs the 16 steps from the
//    true start state and accumulates y += C h.
//  - The chunk's outputs go through LDS and leave as coalesced row segments.  With several
//    directions, partial sums are kept in an fp32 workspace row-aligned with y; the last
//    direction adds, gates and writes y once.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "selscan.h"

namespace {

constexpr int kN = 16;                 // d_state supported by this version
constexpr int kK = 16;                 // consecutive scan steps per lane
constexpr int kLPR = 16;               // lanes per channel: one 16-lane DPP row, 4 channels per wave
constexpr int kCH = kLPR * kK;         // scan steps per chunk (256)
constexpr int kFP = kCH + 4;           // fp32 LDS pitch (floats) of the B, C and y tiles
constexpr int kTC = 16;                // channels per workgroup tile: 4 waves x 4 channels
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

thread_local char g_last_hip_error[160] = "no error";

// ------------------------------------------------------------------------------------
// host-side validation (pure host code: runs before any HIP call)
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

struct Problem {
    const void *x, *delta, *B, *C, *z;
    const float *A, *D, *bias;
    void *y;
    void *ws;
    int64_t batch, L, dim, H, W;
    int ndir;   // 1, 2 or 4
    int kind;   // SELSCAN_OP_*
    int dtype;  // SELSCAN_F32 / SELSCAN_BF16
    unsigned flags;
    const float *h0 = nullptr;  // [batch][dim][N] initial state (forward scan only)
    float *hlast = nullptr;     // [batch][dim][N] state after the last step
    float *ckpt = nullptr;      // [ndir][batch][nchunks][dim][N] state entering each chunk
    int64_t win = 0;            // window side of the windowed cross-scan
};

__host__ __device__ inline int64_t chunks_of(int64_t L) { return (L + kCH - 1) / kCH; }
size_t ckpt_bytes_for(int64_t batch, int64_t L, int64_t dim) {
    return (size_t)batch * (size_t)chunks_of(L) * (size_t)dim * kN * sizeof(float);
}

size_t workspace_bytes_for(int op, int64_t batch, int64_t L, int64_t dim) {
    if (op == SELSCAN_OP_FWD) return 0;
    return (size_t)batch * (size_t)L * (size_t)dim * sizeof(float);
}

int validate(const Problem &p, int64_t dstate, size_t ws_bytes) {
    if (p.batch < 0 || p.L < 0 || p.dim < 0 || p.H < 0 || p.W < 0 || dstate < 0) return SELSCAN_E_SHAPE;
    if (p.dtype != SELSCAN_F32 && p.dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (p.flags & ~SELSCAN_FLAG_DELTA_SOFTPLUS) return SELSCAN_E_UNSUPPORTED;
    if (dstate != kN) return SELSCAN_E_UNSUPPORTED;
    if ((p.kind == SELSCAN_OP_SS2D || p.kind == SELSCAN_OP_LOCAL_SS2D) &&
        (p.L > 0x7FFFFFFF || p.H > 0x7FFFFFFF || p.W > 0x7FFFFFFF))
        return SELSCAN_E_UNSUPPORTED;
    if (p.kind == SELSCAN_OP_LOCAL_SS2D && (p.win < 1 || p.H % p.win || p.W % p.win)) return SELSCAN_E_SHAPE;
    if (p.batch == 0 || p.dim == 0) return SELSCAN_OK;
    if (p.L == 0 && !p.hlast) return SELSCAN_OK;  // nothing to scan and no state to write
    if (p.L > 0 && (!p.x || !p.delta || !p.A || !p.B || !p.C || !p.y)) return SELSCAN_E_NULL;
    const size_t s = p.dtype == SELSCAN_BF16 ? 2 : 4;
    const void *io[] = {p.x, p.delta, p.B, p.C, p.z, p.y};
    for (const void *q : io)
        if (q && !aligned(q, s)) return SELSCAN_E_ALIGN;
    const void *f32[] = {p.A, p.D, p.bias};
    for (const void *q : f32)
        if (q && !aligned(q, 4)) return SELSCAN_E_ALIGN;
    const size_t need = workspace_bytes_for(p.kind, p.batch, p.L, p.dim);
    if (need && p.ws && !aligned(p.ws, 4)) return SELSCAN_E_ALIGN;
    const size_t tok = (size_t)p.batch * p.L * p.dim, bc = (size_t)p.batch * p.L * kN;
    const size_t K = (size_t)p.ndir;
    Span y{p.y, tok * s};
    Span in[] = {{p.x, tok * s},
                 {p.delta, K * tok * s},
                 {p.B, K * bc * s},
                 {p.C, K * bc * s},
                 {p.z, tok * s},
                 {p.A, K * (size_t)p.dim * kN * 4},
                 {p.D, K * (size_t)p.dim * 4},
                 {p.bias, K * (size_t)p.dim * 4},
                 {need ? p.ws : nullptr, need}};
    for (const Span &q : in)
        if (overlap(y, q)) return SELSCAN_E_ALIAS;
    if (need) {
        if (!p.ws || ws_bytes < need) return SELSCAN_E_WORKSPACE;
        for (int i = 0; i < 8; ++i)
            if (overlap({p.ws, need}, in[i])) return SELSCAN_E_ALIAS;
    }
    // state in/out: h_last may be h0 itself (in-place update) but must not overlap anything else
    const size_t st = (size_t)p.batch * (size_t)p.dim * kN * 4;
    if ((p.h0 && !aligned(p.h0, 4)) || (p.hlast && !aligned(p.hlast, 4))) return SELSCAN_E_ALIGN;
    const Span h0s{p.h0, st}, hls{p.hlast, st};
    if (overlap(y, h0s) || overlap(y, hls)) return SELSCAN_E_ALIAS;
    for (const Span &q : in)
        if (overlap(hls, q)) return SELSCAN_E_ALIAS;
    if (p.h0 != (const float *)p.hlast && overlap(hls, h0s)) return SELSCAN_E_ALIAS;
    if (p.ckpt) {
        const Span cks{p.ckpt, K * ckpt_bytes_for(p.batch, p.L, p.dim)};
        if (!aligned(p.ckpt, 4)) return SELSCAN_E_ALIGN;
        if (overlap(cks, y) || overlap(cks, h0s) || overlap(cks, hls)) return SELSCAN_E_ALIAS;
        for (const Span &q : in)
            if (overlap(cks, q)) return SELSCAN_E_ALIAS;
    }
    return SELSCAN_OK;
}

// ------------------------------------------------------------------------------------
// device side
// ------------------------------------------------------------------------------------

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
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    return f.d <= 1 ? n : __umulhi(n, f.m) >> f.sh;
}

struct Params {
    const void *x, *delta, *B, *C, *z;
    const float *A, *D, *bias;
    void *y;
    float *ws;        // fp32 [batch][L][dim] partial sums when ndir > 1
    const float *h0;  // fp32 [batch][dim][N] initial state, or NULL (zero)
    float *hlast;     // fp32 [batch][dim][N] final state, or NULL (not written)
    float *ckpt;      // fp32 [ndir][batch][nchunks][dim][N] state entering each chunk, or NULL
    int64_t L, dim;
    int H, Wd;        // SS2D image height and width (H * Wd == L)
    int win;          // window side of the windowed cross-scan
    FastDiv dH;       // division by H (SS2D column-major order)
    FastDiv dWin, dWin2, dNx, dNy;  // by w, w*w, W/w, H/w (windowed orders)
    int batch, ndir, softplus;
    int vec;          // rows of 8 channels may be moved as 16-byte vectors
    int vecbc;        // a 16-value B/C row may be moved as 16-byte vectors
    int ntc;          // channel tiles per batch row
};

template <typename T>
struct Io;
template <>
struct Io<float> {
    static constexpr int kPadE = 4;  // 16 bytes of padding per lane segment
    __device__ static float f32(float v) { return v; }
    __device__ static float to(float v) { return v; }
};
template <>
struct Io<uint16_t> {
    static constexpr int kPadE = 8;
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

// Shared-memory layout of a workgroup (16 channels), per chunk of kCH steps.  In every tile
// row the 16 steps of a lane are stored as 16-byte pieces: piece q of lane l sits at
// q * (16 lanes * piece) + l * piece, so that one 16-byte read by each of the 16 lanes of a
// row covers 256 contiguous bytes (no bank conflicts).
template <typename T>
struct Lds {
    static constexpr int kCT = kTC;                                  // channels per tile
    static constexpr int kV = 16 / (int)sizeof(T);                    // io elements per piece
    static constexpr int kXP = kCH + kV;                              // io tile pitch (elements)
    static constexpr int kIoBytes = kCT * kXP * (int)sizeof(T);       // x or delta tile
    static constexpr int kYBytes = kCT * kFP * 4;                     // y tile fp32
    // bf16 io: the y tile has space of its own, so a wave writes its outputs without waiting
    // for the other waves to finish reading x and delta.  fp32 io: y reuses the x/delta space
    // (space of its own would leave room for only one workgroup per compute unit).
    static constexpr bool kYOwn = sizeof(T) == 2;
    static constexpr int kXD = 2 * kIoBytes;
    static constexpr int kY = kYOwn ? kXD : 0;
    static constexpr int kB = kYOwn ? kXD + kYBytes : (kXD > kYBytes ? kXD : kYBytes);  // B [state][step]
    static constexpr int kC = kB + kN * kFP * 4;                      // C tile
    static constexpr int kA = kC + kN * kFP * 4;                      // A*log2e [ch][state]
    static constexpr int kCarry = kA + kCT * kN * 4;                  // chunk carry [ch][state]
    static constexpr int kDb = kCarry + kCT * kN * 4;                 // D, bias [ch][2]
    static constexpr int kBytes = kDb + kCT * 8;
    // position of chunk step s in an io tile row
    __device__ static int xpos(int s) { return ((s & 15) / kV) * (kLPR * kV) + (s >> 4) * kV + (s % kV); }
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

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations only.  A
// __syncthreads would also wait for every global load and store the wave has in flight (its
// release fence drains vmcnt), which stalls on stores issued just before the barrier and on
// loads issued for the next chunk.  Within one scan direction no wave reads back global memory
// another wave of the workgroup wrote, so LDS ordering is all these barriers have to give; the
// barrier between directions (where the partial sums change hands) stays a full one.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// softplus(w) = log(1 + e^w) without overflow
__device__ __forceinline__ float softplus(float w) { return w > 0.f ? w + log1pf(__expf(-w)) : log1pf(__expf(w)); }

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

__device__ __forceinline__ void load_f8(const float *p, int n, bool vec, float v[8]) {
    if (vec && n >= 8) {
        const float4 q = *(const float4 *)p, q2 = *(const float4 *)(p + 4);
        v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w, v[4] = q2.x, v[5] = q2.y, v[6] = q2.z, v[7] = q2.w;
        return;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < n ? p[e] : 0.f;
}

// Inclusive scan of two states' lane maps (a, b) along each 16-lane row (one channel):
// (a_l, b_l) <- (a_l a_{l-s}, a_l b_{l-s} + b_l) for s = 1, 2, 4, 8 with DPP row_shr; a lane
// whose source is outside its row is not written, i.e. composed with the identity (1, 0).
// Then every lane's start state: h enters holding the channel's carry and row_shr:1 overwrites
// it with the left neighbour's end state everywhere except in lane 0 of the row, whose source
// is out of range.  The two states alternate so that every DPP read comes at least two wait
// states after the write of its source (the gfx9 VALU->DPP hazard); s_nop covers the ends.
__device__ __forceinline__ void scan16x2(float &b0, float &b1, float &a0, float &a1, float &h0, float &h1) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %2 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %3 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %2, %2 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %3, %3 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %2 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %3 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %2, %2 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %3, %3 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %2 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %3 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %2, %2 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %3, %3 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %0, %2 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %3 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_mov_b32_dpp %4, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mov_b32_dpp %5, %1 row_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(b0), "+v"(b1), "+v"(a0), "+v"(a1), "+v"(h0), "+v"(h1));
}

// One workgroup: 4 waves, a tile of 16 channels of one batch row, every direction.
//
// Lane maps of the staging and output items (wave w, lane i of the wave) are chosen so that
// each LDS write or read instruction of a wave touches 64 distinct banks:
//  - x/delta staging: chunk steps 2p, 2p+1 of the 8-channel group g = i / 32, with
//    p = 8 (((i / 4) % 8) + 8 (w / 2)) + 4 (w % 2) + i % 4;
//  - B/C staging: chunk step 16 (i / 4) + 4 w + i % 4, all 16 states;
//  - output: chunk steps 16 ((i / 4) % 8 + 8 r) + 4 w + i % 4, r = 0, 1, group g = i / 32.
// Priority: the waves of the two workgroups that share a SIMD run their state loops at
// priorities that alternate with the chunk count, so neither workgroup starves the other,
// and every phase outside the state loop runs above both.
template <typename T, int KIND>
__global__ __launch_bounds__(256, 2) void selscan_chunked(Params p) {
    using S = Lds<T>;
    constexpr int CT = kTC;
    constexpr int NW = kN * (int)sizeof(T) / 4;  // dwords of one 16-value B or C row
    static_assert(CT * kN == 256, "one (channel, state) carry entry per thread");
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::kBytes];
    T *xt = (T *)smem;
    T *dtl = (T *)(smem + S::kIoBytes);
    float *yt = (float *)(smem + S::kY);
    float *Bs = (float *)(smem + S::kB);
    float *Cs = (float *)(smem + S::kC);
    float *As = (float *)(smem + S::kA);
    float *Cy = (float *)(smem + S::kCarry);
    float *Db = (float *)(smem + S::kDb);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l = lane & 15;
    const int cl = wave * 4 + (lane >> 4);     // this lane's channel within the tile
    const float firstf = l == 0 ? 1.f : 0.f;  // 1 on the first lane of each channel
    // consecutive channel tiles on one XCD: workgroups are dealt round-robin over 8 XCDs
    const int G = gridDim.x, bi = blockIdx.x, q8 = G >> 3;
    const int tile = bi < (q8 << 3) ? (bi & 7) * q8 + (bi >> 3) : bi;
    const int b = tile / p.ntc;
    const int64_t c0 = (int64_t)(tile % p.ntc) * CT;
    const int64_t L = p.L, dim = p.dim;
    const int64_t tok = (int64_t)p.batch * L * dim, bcn = (int64_t)p.batch * L * kN;
    const int ncols = (int)(dim - c0 < CT ? dim - c0 : CT);
    const bool cvalid = cl < ncols;
    const int nchunks = (int)((L + kCH - 1) / kCH);
    const bool tile_fast = ncols == CT && p.vec && p.vecbc;  // full tile, vector rows
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x;
    const T *z = (const T *)p.z;
    T *y = (T *)p.y;
    const int64_t rowb = (int64_t)b * L;

    const int g = lane >> 5, nv = ncols - 8 * g;  // 8-channel group of the row items
    const int64_t cg = c0 + 8 * g;
    const int pp = 8 * (((lane >> 2) & 7) + 8 * (wave >> 1)) + 4 * (wave & 1) + (lane & 3);
    const int sb = 16 * (lane >> 2) + 4 * wave + (lane & 3);
    const int so = 16 * ((lane >> 2) & 7) + 4 * wave + (lane & 3);

    int qq = 0;  // chunks done over all directions (priority parity)
    for (int k = 0; k < p.ndir; ++k) {
        const T *dl = (const T *)p.delta + k * tok;
        const T *Bk = (const T *)p.B + k * bcn;
        const T *Ck = (const T *)p.C + k * bcn;
        // the previous direction is done with the parameter tiles, and its stores of the partial
        // sums (which other waves read back in this direction) are complete: a full barrier
        __syncthreads();
        for (int i = tid; i < CT * kN; i += 256) {
            const int ch = i / kN, n = i % kN;
            const int64_t cc = c0 + ch < dim ? c0 + ch : 0;
            if (nchunks > 0) As[i] = p.A[(k * dim + cc) * kN + n] * kLog2e;
            // the carry into the first chunk: the caller's initial state, else zero
            Cy[i] = p.h0 && c0 + ch < dim ? p.h0[((int64_t)b * dim + c0 + ch) * kN + n] : 0.f;
        }
        for (int i = tid; i < CT && nchunks > 0; i += 256) {
            const int64_t cc = c0 + i < dim ? c0 + i : 0;
            Db[2 * i] = p.D ? p.D[k * dim + cc] : 0.f;
            Db[2 * i + 1] = p.bias ? p.bias[k * dim + cc] : 0.f;
        }

        // global -> registers for chunk q (prefetched one chunk ahead)
        Raw8<T> px0, px1, pd0, pd1;
        uint32_t pbc[2][NW];  // raw B and C values of one chunk step
        auto fetch = [&](int q, auto fast_c) {
            const int64_t s0 = (int64_t)q * kCH;
            const int64_t sa = s0 + 2 * pp, sbb = sa + 1, s = s0 + sb;
            if constexpr (decltype(fast_c)::value) {
                const int64_t oa = (rowb + visit<KIND>(p, k, sa)) * dim + cg;
                const int64_t ob = (rowb + visit<KIND>(p, k, sbb)) * dim + cg;
                px0 = load_raw8(x + oa, 8, true);
                pd0 = load_raw8(dl + oa, 8, true);
                px1 = load_raw8(x + ob, 8, true);
                pd1 = load_raw8(dl + ob, 8, true);
                const int64_t ro = (rowb + visit<KIND>(p, k, s)) * kN;
#pragma unroll
                for (int h = 0; h < NW; h += 4) {
                    const uint4 qb = *(const uint4 *)((const uint32_t *)(Bk + ro) + h);
                    const uint4 qc = *(const uint4 *)((const uint32_t *)(Ck + ro) + h);
                    pbc[0][h] = qb.x, pbc[0][h + 1] = qb.y, pbc[0][h + 2] = qb.z, pbc[0][h + 3] = qb.w;
                    pbc[1][h] = qc.x, pbc[1][h + 1] = qc.y, pbc[1][h + 2] = qc.z, pbc[1][h + 3] = qc.w;
                }
            } else {
                px0 = px1 = pd0 = pd1 = Raw8<T>{};
                if (nv > 0 && sa < L) {
                    const int64_t off = (rowb + visit<KIND>(p, k, sa)) * dim + cg;
                    px0 = load_raw8(x + off, nv, vec);
                    pd0 = load_raw8(dl + off, nv, vec);
                }
                if (nv > 0 && sbb < L) {
                    const int64_t off = (rowb + visit<KIND>(p, k, sbb)) * dim + cg;
                    px1 = load_raw8(x + off, nv, vec);
                    pd1 = load_raw8(dl + off, nv, vec);
                }
#pragma unroll
                for (int h = 0; h < NW; ++h) pbc[0][h] = pbc[1][h] = 0u;
                if (s < L) {
                    const int64_t ro = (rowb + visit<KIND>(p, k, s)) * kN;
                    if (p.vecbc) {
#pragma unroll
                        for (int h = 0; h < NW; h += 4) {
                            const uint4 qb = *(const uint4 *)((const uint32_t *)(Bk + ro) + h);
                            const uint4 qc = *(const uint4 *)((const uint32_t *)(Ck + ro) + h);
                            pbc[0][h] = qb.x, pbc[0][h + 1] = qb.y, pbc[0][h + 2] = qb.z, pbc[0][h + 3] = qb.w;
                            pbc[1][h] = qc.x, pbc[1][h + 1] = qc.y, pbc[1][h + 2] = qc.z, pbc[1][h + 3] = qc.w;
                        }
                    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
                        for (int h = 0; h < NW; ++h) {
                            pbc[0][h] = (uint32_t)Bk[ro + 2 * h] | ((uint32_t)Bk[ro + 2 * h + 1] << 16);
                            pbc[1][h] = (uint32_t)Ck[ro + 2 * h] | ((uint32_t)Ck[ro + 2 * h + 1] << 16);
                        }
                    } else {
#pragma unroll
                        for (int h = 0; h < NW; ++h) {
                            pbc[0][h] = __float_as_uint(Bk[ro + h]);
                            pbc[1][h] = __float_as_uint(Ck[ro + h]);
                        }
                    }
                }
            }
        };
        // registers -> LDS
        auto commit = [&]() {
            const int si = S::xpos(2 * pp);  // steps 2p and 2p+1 are adjacent in a piece
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ch = 8 * g + e;
                if constexpr (sizeof(T) == 2) {
                    // low half: step 2p, high half: step 2p+1, of channel e (v_perm_b32)
                    const uint32_t sel = e & 1 ? 0x07060302u : 0x05040100u;
                    *(uint32_t *)&xt[ch * S::kXP + si] = __builtin_amdgcn_perm(px1.w[e >> 1], px0.w[e >> 1], sel);
                    *(uint32_t *)&dtl[ch * S::kXP + si] = __builtin_amdgcn_perm(pd1.w[e >> 1], pd0.w[e >> 1], sel);
                } else {
                    *(uint2 *)&xt[ch * S::kXP + si] = make_uint2(px0.w[e], px1.w[e]);
                    *(uint2 *)&dtl[ch * S::kXP + si] = make_uint2(pd0.w[e], pd1.w[e]);
                }
            }
            const int sp = fpos(sb);
#pragma unroll
            for (int h = 0; h < kN; ++h) {
                float bv, cv;
                if constexpr (sizeof(T) == 2) {
                    bv = __uint_as_float(h & 1 ? pbc[0][h >> 1] & 0xFFFF0000u : pbc[0][h >> 1] << 16);
                    cv = __uint_as_float(h & 1 ? pbc[1][h >> 1] & 0xFFFF0000u : pbc[1][h >> 1] << 16);
                } else {
                    bv = __uint_as_float(pbc[0][h]);
                    cv = __uint_as_float(pbc[1][h]);
                }
                Bs[h * kFP + sp] = bv;
                Cs[h * kFP + sp] = cv;
            }
        };

        // one chunk; FAST: a full chunk of a full tile whose successor is full too
        auto chunk = [&](int q, auto fast_c) {
            constexpr bool fast = decltype(fast_c)::value;
            const int64_t s0 = (int64_t)q * kCH;
            __builtin_amdgcn_s_setprio(2);
            lds_barrier();  // the previous chunk is done with every tile
            commit();
            lds_barrier();
            if (p.ckpt) {
                // the carry entering this chunk, kept for the backward pass
                const int ch = tid / kN, n = tid % kN;
                if (c0 + ch < dim)
                    p.ckpt[((((int64_t)k * p.batch + b) * nchunks + q) * dim + c0 + ch) * kN + n] = Cy[tid];
            }
            // gate input for this chunk's output items, then the next chunk's inputs: in flight
            // while this chunk computes
            const bool last = k == p.ndir - 1;
            Raw8<T> zr[2] = {};
            int64_t ooff[2] = {0, 0};
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int64_t s = s0 + so + 128 * r;
                if constexpr (fast) {
                    ooff[r] = (rowb + visit<KIND>(p, k, s)) * dim + cg;
                    if (last && z) zr[r] = load_raw8(z + ooff[r], 8, true);
                } else if (nv > 0 && s < L) {
                    ooff[r] = (rowb + visit<KIND>(p, k, s)) * dim + cg;
                    if (last && z) zr[r] = load_raw8(z + ooff[r], nv, vec);
                }
            }
            if (q + 1 < nchunks) fetch(q + 1, fast_c);

            // ---- this lane's 16 steps of its channel
            const int64_t rem = L - (s0 + l * kK);
            const int lim = !cvalid ? 0 : (rem <= 0 ? 0 : (rem >= kK ? kK : (int)rem));
            float dt[kK], dx[kK], yv[kK];
            float sdt = 0.f;
            {
                const float Dd = Db[2 * cl], bias = Db[2 * cl + 1];
                float xf[kK], df[kK];
                constexpr int V = S::kV;
#pragma unroll
                for (int pc = 0; pc < kK / V; ++pc) {
                    const uint4 xq = *(const uint4 *)&xt[cl * S::kXP + pc * (kLPR * V) + l * V];
                    const uint4 dq = *(const uint4 *)&dtl[cl * S::kXP + pc * (kLPR * V) + l * V];
                    const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w}, dw[4] = {dq.x, dq.y, dq.z, dq.w};
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        if constexpr (sizeof(T) == 2) {
                            xf[pc * V + i] = __uint_as_float(i & 1 ? xw[i >> 1] & 0xFFFF0000u : xw[i >> 1] << 16);
                            df[pc * V + i] = __uint_as_float(i & 1 ? dw[i >> 1] & 0xFFFF0000u : dw[i >> 1] << 16);
                        } else {
                            xf[pc * V + i] = __uint_as_float(xw[i]);
                            df[pc * V + i] = __uint_as_float(dw[i]);
                        }
                    }
                }
                if (p.softplus) {
#pragma unroll
                    for (int j = 0; j < kK; ++j) dt[j] = softplus(df[j] + bias);
                } else {
#pragma unroll
                    for (int j = 0; j < kK; ++j) dt[j] = df[j] + bias;
                }
                if (!fast && !(s0 + kCH <= L && ncols == CT)) {
                    // steps past the sequence end and channels past dim get delta = 0, the
                    // identity step (staged x there is 0 too)
                    const float limf = (float)lim;
#pragma unroll
                    for (int j = 0; j < kK; ++j) dt[j] *= __saturatef(limf - (float)j);
                }
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    dx[j] = dt[j] * xf[j];
                    yv[j] = Dd * xf[j];
                    sdt += dt[j];
                }
            }
            if (qq & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            const float *Bc = Bs + 4 * l;
            const float *Cc = Cs + 4 * l;
#pragma unroll 1
            for (int n = 0; n < kN; n += 2) {
                const float2 a2 = *(const float2 *)&As[cl * kN + n];
                float e0[kK], u0[kK], e1[kK], u1[kK];
                float b0, b1;
                {
                    float B0[kK], B1[kK];
#pragma unroll
                    for (int pc = 0; pc < 4; ++pc) {
                        *(float4 *)&B0[4 * pc] = *(const float4 *)&Bc[n * kFP + pc * (kLPR * 4)];
                        *(float4 *)&B1[4 * pc] = *(const float4 *)&Bc[(n + 1) * kFP + pc * (kLPR * 4)];
                    }
#pragma unroll
                    for (int j = 0; j < kK; ++j) {
                        e0[j] = __builtin_amdgcn_exp2f(dt[j] * a2.x);
                        e1[j] = __builtin_amdgcn_exp2f(dt[j] * a2.y);
                        u0[j] = dx[j] * B0[j];
                        u1[j] = dx[j] * B1[j];
                        b0 = j == 0 ? u0[0] : fmaf(e0[j], b0, u0[j]);  // from a zero state
                        b1 = j == 0 ? u1[0] : fmaf(e1[j], b1, u1[j]);
                    }
                }
                float a0 = __builtin_amdgcn_exp2f(a2.x * sdt);
                float a1 = __builtin_amdgcn_exp2f(a2.y * sdt);
                // the previous chunk's end state of this channel enters through its first lane
                const float2 cy = *(const float2 *)&Cy[cl * kN + n];
                float h0 = cy.x, h1 = cy.y;
                b0 = fmaf(a0, h0 * firstf, b0);
                b1 = fmaf(a1, h1 * firstf, b1);
                scan16x2(b0, b1, a0, a1, h0, h1);
                // the last lane of a channel holds the chunk's end state: the next chunk's carry
                if (l == kLPR - 1) *(float2 *)&Cy[cl * kN + n] = make_float2(b0, b1);
                float C0[kK], C1[kK];
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) {
                    *(float4 *)&C0[4 * pc] = *(const float4 *)&Cc[n * kFP + pc * (kLPR * 4)];
                    *(float4 *)&C1[4 * pc] = *(const float4 *)&Cc[(n + 1) * kFP + pc * (kLPR * 4)];
                }
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    h0 = fmaf(e0[j], h0, u0[j]);
                    h1 = fmaf(e1[j], h1, u1[j]);
                    yv[j] = fmaf(C0[j], h0, yv[j]);
                    yv[j] = fmaf(C1[j], h1, yv[j]);
                }
            }
            __builtin_amdgcn_s_setprio(2);
            if constexpr (!S::kYOwn) lds_barrier();  // x/delta tiles fully read before y reuses their space
#pragma unroll
            for (int pc = 0; pc < 4; ++pc)
                *(float4 *)&yt[cl * kFP + pc * (kLPR * 4) + 4 * l] =
                    make_float4(yv[4 * pc], yv[4 * pc + 1], yv[4 * pc + 2], yv[4 * pc + 3]);
            lds_barrier();
            // ---- leave: add earlier directions, gate, store y (or keep the partial sum)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int sl = so + 128 * r;
                float v[8], wv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if constexpr (fast) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = yt[(8 * g + e) * kFP + fpos(sl)];
                    if (k > 0) load_f8(p.ws + ooff[r], 8, true, wv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += wv[e];
                    if (last) {
                        if (z) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] *= silu(raw_f32(zr[r], e));
                        }
                        store8(y + ooff[r], 8, true, v);
                    } else {
                        store8(p.ws + ooff[r], 8, true, v);
                    }
                } else if (nv > 0 && s0 + sl < L) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = yt[(8 * g + e) * kFP + fpos(sl)];
                    if (k > 0) load_f8(p.ws + ooff[r], nv, vec, wv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += wv[e];
                    if (last) {
                        if (z) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] *= silu(raw_f32(zr[r], e));
                        }
                        store8(y + ooff[r], nv, vec, v);
                    } else {
                        store8(p.ws + ooff[r], nv, vec, v);
                    }
                }
            }
        };
        fetch(0, BoolC<false>{});
        const int nfast = tile_fast ? (int)(L / kCH) - 1 : 0;
        int q = 0;
        for (; q < nfast; ++q, ++qq) chunk(q, BoolC<true>{});
        for (; q < nchunks; ++q, ++qq) chunk(q, BoolC<false>{});
    }
    if (p.hlast) {
        // the last chunk's carry is the state after step L-1 (steps past L are identity steps)
        lds_barrier();
        for (int i = tid; i < CT * kN; i += 256) {
            const int ch = i / kN, n = i % kN;
            if (c0 + ch < dim) p.hlast[((int64_t)b * dim + c0 + ch) * kN + n] = Cy[i];
        }
    }
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

template <typename T, int KIND>
int launch_tiles(const Params &a, int64_t batch, void *stream) {
    Params c = a;
    c.ntc = (int)((a.dim + kTC - 1) / kTC);
    const int64_t blocks = batch * (int64_t)c.ntc;
    if (blocks > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    void *args[] = {&c};
    hipError_t e = hipLaunchKernel((const void *)&selscan_chunked<T, KIND>, dim3((unsigned)blocks), dim3(256),
                                   args, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
        return SELSCAN_E_HIP;
    }
    return SELSCAN_OK;
}

template <typename T>
int launch_kind(const Params &a, int kind, int64_t batch, void *stream) {
    if (kind == SELSCAN_OP_FWD) return launch_tiles<T, SELSCAN_OP_FWD>(a, batch, stream);
    if (kind == SELSCAN_OP_BIDIR) return launch_tiles<T, SELSCAN_OP_BIDIR>(a, batch, stream);
    if (kind == SELSCAN_OP_SS2D) return launch_tiles<T, SELSCAN_OP_SS2D>(a, batch, stream);
    return launch_tiles<T, SELSCAN_OP_LOCAL_SS2D>(a, batch, stream);
}

int launch(const Problem &p, void *stream) {
    Params a;
    a.x = p.x, a.delta = p.delta, a.B = p.B, a.C = p.C, a.z = p.z;
    a.A = p.A, a.D = p.D, a.bias = p.bias, a.y = p.y;
    a.ws = p.ndir > 1 ? (float *)p.ws : nullptr;
    a.h0 = p.h0, a.hlast = p.hlast, a.ckpt = p.ckpt;
    a.dim = p.dim;
    set_order(a, p.kind, p.L, p.H, p.W, p.win);
    a.batch = (int)p.batch, a.ndir = p.ndir;
    a.softplus = (p.flags & SELSCAN_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
    // rows of 8 channels move as 16-byte vectors when every row start is 16-byte aligned
    const void *rows[] = {p.x, p.delta, p.z, p.y};
    bool vec = p.dim % 8 == 0 && (!a.ws || aligned(a.ws, 16));
    for (const void *q : rows)
        if (q && !aligned(q, 16)) vec = false;
    a.vec = vec;
    a.vecbc = aligned(p.B, 16) && aligned(p.C, 16);
    a.ntc = 0;
    if (p.dtype == SELSCAN_BF16) return launch_kind<uint16_t>(a, p.kind, p.batch, stream);
    return launch_kind<float>(a, p.kind, p.batch, stream);
}

int run(Problem &p, int64_t dstate, size_t ws_bytes, void *stream) {
    int rc = validate(p, dstate, ws_bytes);
    if (rc != SELSCAN_OK) return rc;
    if (p.batch == 0 || p.dim == 0 || (p.L == 0 && !p.hlast)) return SELSCAN_OK;
    if (p.batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    return launch(p, stream);
}

// ------------------------------------------------------------------------------------
// backward of the single-direction scan
// ------------------------------------------------------------------------------------
//
// Reverse-mode derivative of selscan_fwd (Euler Bbar), recomputing the states chunk by chunk
// from the last chunk back, each chunk starting from the state the forward saved on entering
// it (the states are recomputed in the backward instead of stored: "Mamba论文" and "Mamba
// Series ..." section 核心洞察).  With e_t = exp(delta_t A), u_t = delta_t B_t x_t,
// h_t = e_t h_{t-1} + u_t, dyp_t = dy_t silu(z_t) and g_t = dL/dh_t (total derivative):
//   g_t = C_t dyp_t + e_{t+1} g_{t+1}.
// Written for gt_t = e_t g_t (what step t hands to h_{t-1}): g_t = C_t dyp_t + gt_{t+1},
// gt_t = e_t g_t -- an affine recurrence running down in time with the forward's own decay,
// so each lane folds its 16 steps into a map and the maps are scanned across the 16 lanes of
// the channel towards lane 0 (DPP row_shl), the mirror of the forward scan.  Per (t, n):
//   ddelta_t += g_t (A e_t h_{t-1} + B_t x_t),   dA += g_t delta_t e_t h_{t-1},
//   dx_t += g_t delta_t B_t,   dB_t += g_t delta_t x_t,   dC_t += dyp_t h_t,
// with e_t h_{t-1} = h_t - u_t and B_t x_t = u_t / delta_t.  dB and dC are summed over the
// tile's 16 channels (v_permlane32/16_swap across the 4 channel rows of a wave, then LDS
// across the 4 waves) and leave as one fp32 partial per tile; selscan_bwd_reduce adds the
// tiles and the batch rows.
//
// Several directions (bidirectional, SS2D, windowed): the merged output is
// y = (sum_k o_k) silu(z), each o_k a single-direction scan on its own visiting order, so
// direction k's backward is the one above with dL/do_k = dy silu(z) at the pixels it visits.
// The workgroup walks the directions one after another, as the forward does; dx (summed over
// the directions) and the pre-gate output sum_k o_k (which dz needs) build up in fp32 rows
// of the workspace, and the last direction writes dx and dz.

struct BwdParams {
    const void *x, *delta, *B, *C, *z, *dy;
    const float *A, *D, *bias, *ckpt;
    void *dx, *ddelta, *dz;
    float *dh0;
    float *wsBC;  // [ndir][ntc][batch][2][N][L] per-tile partial sums of dB (0) and dC (1), by scan step
    float *wsA;   // [ndir][batch][dim][N] per-batch-row partial sums of dA
    float *wsD;   // [ndir][batch][dim][2] per-batch-row partial sums of dD and ddelta_bias
    float *wsX;   // [batch][L][dim] dx summed over the directions done so far (ndir > 1)
    float *wsY;   // [batch][L][dim] pre-gate output summed over the directions done so far (ndir > 1)
    int64_t L, dim;
    int H, Wd, win;  // scan order (as for the forward)
    FastDiv dH, dWin, dWin2, dNx, dNy;
    int batch, ndir, softplus, ntc, vec, vecbc;
};

// Shared memory of one backward workgroup (16 channels, one chunk).
template <typename T>
struct BwdLds {
    static constexpr int kV = 16 / (int)sizeof(T);
    static constexpr int kXP = kCH + kV;
    static constexpr int kIo = kTC * kXP * (int)sizeof(T);  // one io tile
    static constexpr int kX = 0, kDl = kIo, kDy = 2 * kIo, kZ = 3 * kIo;
    static constexpr int kB = 4 * kIo;                      // fp32 [state][step]
    static constexpr int kC = kB + kN * kFP * 4;
    static constexpr int kA = kC + kN * kFP * 4;            // A*log2e [ch][state]
    static constexpr int kHc = kA + kTC * kN * 4;           // state entering the chunk
    static constexpr int kGc = kHc + kTC * kN * 4;          // adjoint carried to the earlier chunk
    static constexpr int kDA = kGc + kTC * kN * 4;          // dA accumulated over the chunks
    static constexpr int kDb = kDA + kTC * kN * 4;          // D, bias [ch][2]
    static constexpr int kDD = kDb + kTC * 8;               // dD, dbias accumulated [ch][2]
    static constexpr int kBytes = kDD + kTC * 8;
    // the x tile is dead after the prologue: it holds the channel-sum buffers of dB, dC
    static constexpr int kRed = kX;                         // fp32 [2][4 waves][256]
    static_assert(2 * 4 * kCH * 4 <= kIo, "reduction buffer fits in the x tile");
    __device__ static int xpos(int s) { return ((s & 15) / kV) * (kLPR * kV) + (s >> 4) * kV + (s % kV); }
};

// Inclusive scan of one state's lane maps along each 16-lane row.  Up: towards higher lanes
// (lane l composes with l-s), then h <- the left neighbour's b (lane 0 keeps h).  Down: the
// mirror (lane l composes with l+s, h <- the right neighbour's b, lane 15 keeps h).  One
// state at a time, so every DPP read waits two states after the write of its source.
__device__ __forceinline__ void scan16_up(float &b, float &a, float &h) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_mov_b32_dpp %2, %0 row_shr:1 row_mask:0xf bank_mask:0xf"
        : "+v"(b), "+v"(a), "+v"(h));
}
__device__ __forceinline__ void scan16_down(float &b, float &a, float &h) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shl:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shl:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %1, %1 row_shl:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %1 row_shl:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_mov_b32_dpp %2, %0 row_shl:1 row_mask:0xf bank_mask:0xf"
        : "+v"(b), "+v"(a), "+v"(h));
}

// Sum over the 16 lanes of each row; the total lands in lane 15 of the row.
__device__ __forceinline__ float rowsum16(float v) {
    asm volatile(
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_add_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v));
    return v;
}

// 16 per-step values of each lane -> 4 registers holding, in row r of register k, the sum
// over the wave's 4 channel rows of step k + 4 r of the lane (v_permlane32_swap pairs the
// upper and lower half-waves, v_permlane16_swap the odd and even rows).
__device__ __forceinline__ void rows4_sum(const float p[kK], float out[4]) {
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[j]), __float_as_uint(p[j + 8]), false,
                                                       false);
        s[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[k]), __float_as_uint(s[k + 4]), false,
                                                       false);
        out[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

__device__ __forceinline__ float sigmoidf_(float w) { return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-w * kLog2e)); }

template <typename T, int KIND>
__global__ __launch_bounds__(256, 2) void selscan_bwd_chunked(BwdParams p) {
    constexpr bool multi = KIND != SELSCAN_OP_FWD;
    using S = BwdLds<T>;
    constexpr int CT = kTC;
    static_assert(CT * kN == 256, "one (channel, state) entry per thread");
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::kBytes];
    T *xt = (T *)(smem + S::kX);
    T *dtl = (T *)(smem + S::kDl);
    T *dyt = (T *)(smem + S::kDy);
    T *zt = (T *)(smem + S::kZ);
    float *Bs = (float *)(smem + S::kB);
    float *Cs = (float *)(smem + S::kC);
    float *As = (float *)(smem + S::kA);
    float *Hc = (float *)(smem + S::kHc);
    float *Gc = (float *)(smem + S::kGc);
    float *dAs = (float *)(smem + S::kDA);
    float *Db = (float *)(smem + S::kDb);
    float *dDs = (float *)(smem + S::kDD);
    float *red = (float *)(smem + S::kRed);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l = lane & 15, row = lane >> 4;
    const int cl = wave * 4 + row;
    const float firstf = l == 0 ? 1.f : 0.f, lastf = l == kLPR - 1 ? 1.f : 0.f;
    const int G = gridDim.x, bi = blockIdx.x, q8 = G >> 3;
    const int tile = bi < (q8 << 3) ? (bi & 7) * q8 + (bi >> 3) : bi;
    const int b = tile / p.ntc, tc = tile % p.ntc;
    const int64_t c0 = (int64_t)tc * CT;
    const int64_t L = p.L, dim = p.dim;
    const int ncols = (int)(dim - c0 < CT ? dim - c0 : CT);
    const bool cvalid = cl < ncols;
    const int nchunks = (int)chunks_of(L);
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x;
    const T *dy = (const T *)p.dy;
    const T *z = (const T *)p.z;
    const int64_t rowb = (int64_t)b * L;
    const int64_t tok = (int64_t)p.batch * L * dim, bcn = (int64_t)p.batch * L * kN;
    const int g = lane >> 5, nv = ncols - 8 * g;
    const int64_t cg = c0 + 8 * g;
    const int pp = 8 * (((lane >> 2) & 7) + 8 * (wave >> 1)) + 4 * (wave & 1) + (lane & 3);
    const int sb = 16 * (lane >> 2) + 4 * wave + (lane & 3);
    const int so = 16 * ((lane >> 2) & 7) + 4 * wave + (lane & 3);
    constexpr int NW = kN * (int)sizeof(T) / 4;

  const int ndir = multi ? p.ndir : 1;
  for (int k = 0; k < ndir; ++k) {
    const T *dl = (const T *)p.delta + k * tok;
    const T *Bg = (const T *)p.B + k * bcn;
    const T *Cg = (const T *)p.C + k * bcn;
    const bool last = k == ndir - 1;
    // the previous direction is done with every tile, and its stores of the summed rows (read
    // back here by other waves) are complete: a full barrier
    __syncthreads();
    {
        const int ch = tid / kN, n = tid % kN;
        const int64_t cc = c0 + ch < dim ? c0 + ch : 0;
        As[tid] = nchunks > 0 ? p.A[(k * dim + cc) * kN + n] * kLog2e : 0.f;
        Gc[tid] = 0.f;  // nothing flows back from after the last step
        dAs[tid] = 0.f;
        if (tid < CT) {
            const int64_t c1 = c0 + tid < dim ? c0 + tid : 0;
            Db[2 * tid] = p.D ? p.D[k * dim + c1] : 0.f;
            Db[2 * tid + 1] = p.bias ? p.bias[k * dim + c1] : 0.f;
            dDs[2 * tid] = dDs[2 * tid + 1] = 0.f;
        }
    }

    for (int q = nchunks - 1; q >= 0; --q) {
        const int64_t s0 = (int64_t)q * kCH;
        lds_barrier();  // the previous (later) chunk is done with every tile
        // ---- stage x, delta, dy, z (io) and B, C (fp32); the chunk's entry state
        {
            Raw8<T> r0[4], r1[4];
            const int64_t sa = s0 + 2 * pp, sbb = sa + 1;
            const T *src[4] = {x, dl, dy, z};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                r0[m] = r1[m] = Raw8<T>{};
                if (!src[m]) continue;
                if (nv > 0 && sa < L) r0[m] = load_raw8(src[m] + (rowb + visit<KIND>(p, k, sa)) * dim + cg, nv, vec);
                if (nv > 0 && sbb < L) r1[m] = load_raw8(src[m] + (rowb + visit<KIND>(p, k, sbb)) * dim + cg, nv, vec);
            }
            uint32_t pbc[2][NW];
#pragma unroll
            for (int h = 0; h < NW; ++h) pbc[0][h] = pbc[1][h] = 0u;
            const int64_t s = s0 + sb;
            if (s < L) {
                const int64_t ro = (rowb + visit<KIND>(p, k, s)) * kN;
                if (p.vecbc) {
#pragma unroll
                    for (int h = 0; h < NW; h += 4) {
                        const uint4 qb = *(const uint4 *)((const uint32_t *)(Bg + ro) + h);
                        const uint4 qc = *(const uint4 *)((const uint32_t *)(Cg + ro) + h);
                        pbc[0][h] = qb.x, pbc[0][h + 1] = qb.y, pbc[0][h + 2] = qb.z, pbc[0][h + 3] = qb.w;
                        pbc[1][h] = qc.x, pbc[1][h + 1] = qc.y, pbc[1][h + 2] = qc.z, pbc[1][h + 3] = qc.w;
                    }
                } else if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int h = 0; h < NW; ++h) {
                        pbc[0][h] = (uint32_t)Bg[ro + 2 * h] | ((uint32_t)Bg[ro + 2 * h + 1] << 16);
                        pbc[1][h] = (uint32_t)Cg[ro + 2 * h] | ((uint32_t)Cg[ro + 2 * h + 1] << 16);
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < NW; ++h) {
                        pbc[0][h] = __float_as_uint(Bg[ro + h]);
                        pbc[1][h] = __float_as_uint(Cg[ro + h]);
                    }
                }
            }
            const int si = S::xpos(2 * pp);
            T *dst[4] = {xt, dtl, dyt, zt};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ch = 8 * g + e;
                    if constexpr (sizeof(T) == 2) {
                        const uint32_t sel = e & 1 ? 0x07060302u : 0x05040100u;
                        *(uint32_t *)&dst[m][ch * S::kXP + si] = __builtin_amdgcn_perm(r1[m].w[e >> 1], r0[m].w[e >> 1], sel);
                    } else {
                        *(uint2 *)&dst[m][ch * S::kXP + si] = make_uint2(r0[m].w[e], r1[m].w[e]);
                    }
                }
            }
            const int sp = fpos(sb);
#pragma unroll
            for (int h = 0; h < kN; ++h) {
                float bv, cv;
                if constexpr (sizeof(T) == 2) {
                    bv = __uint_as_float(h & 1 ? pbc[0][h >> 1] & 0xFFFF0000u : pbc[0][h >> 1] << 16);
                    cv = __uint_as_float(h & 1 ? pbc[1][h >> 1] & 0xFFFF0000u : pbc[1][h >> 1] << 16);
                } else {
                    bv = __uint_as_float(pbc[0][h]);
                    cv = __uint_as_float(pbc[1][h]);
                }
                Bs[h * kFP + sp] = bv;
                Cs[h * kFP + sp] = cv;
            }
            const int ch = tid / kN, n = tid % kN;
            Hc[tid] = c0 + ch < dim ? p.ckpt[((((int64_t)k * p.batch + b) * nchunks + q) * dim + c0 + ch) * kN + n]
                                    : 0.f;
        }
        lds_barrier();

        // ---- this lane's 16 steps of its channel
        const int64_t rem = L - (s0 + l * kK);
        const int lim = !cvalid ? 0 : (rem <= 0 ? 0 : (rem >= kK ? kK : (int)rem));
        float dt[kK], dlx[kK], dyp[kK], yv[kK];
        float sdt = 0.f, dDl = 0.f;
        const float Dd = Db[2 * cl], bias = Db[2 * cl + 1];
        {
            float xf[kK], df[kK], yf[kK], zf[kK];
            constexpr int V = S::kV;
            const T *tl[4] = {xt, dtl, dyt, zt};
            float *fl[4] = {xf, df, yf, zf};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int pc = 0; pc < kK / V; ++pc) {
                    const uint4 v4 = *(const uint4 *)&tl[m][cl * S::kXP + pc * (kLPR * V) + l * V];
                    const uint32_t w4[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        if constexpr (sizeof(T) == 2)
                            fl[m][pc * V + i] = __uint_as_float(i & 1 ? w4[i >> 1] & 0xFFFF0000u : w4[i >> 1] << 16);
                        else
                            fl[m][pc * V + i] = __uint_as_float(w4[i]);
                    }
                }
            }
            const float limf = (float)lim;
#pragma unroll
            for (int j = 0; j < kK; ++j) {
                const float w = df[j] + bias;
                dt[j] = (p.softplus ? softplus(w) : w) * __saturatef(limf - (float)j);
                dlx[j] = dt[j] * xf[j];
                dyp[j] = z ? yf[j] * silu(zf[j]) : yf[j];
                yv[j] = Dd * xf[j];
                dDl = fmaf(dyp[j], xf[j], dDl);
                sdt += dt[j];
            }
        }
        float accdd[kK], acc1[kK], accx[kK];
#pragma unroll
        for (int j = 0; j < kK; ++j) accdd[j] = acc1[j] = accx[j] = 0.f;
        const float *Bc = Bs + 4 * l;
        const float *Cc = Cs + 4 * l;
        float *redB = red + wave * kCH, *redC = red + 4 * kCH + wave * kCH;

#pragma unroll 1
        for (int n = 0; n < kN; ++n) {
            const float a2 = As[cl * kN + n];
            const float Araw = a2 * kLn2;
            float e[kK], u[kK], hh[kK], c[kK];
            // forward, pass 1: from a zero state
            float bq;
            {
                float Bv[kK];
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) *(float4 *)&Bv[4 * pc] = *(const float4 *)&Bc[n * kFP + pc * (kLPR * 4)];
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    e[j] = __builtin_amdgcn_exp2f(dt[j] * a2);
                    u[j] = dlx[j] * Bv[j];
                    bq = j == 0 ? u[0] : fmaf(e[j], bq, u[j]);
                }
            }
            const float aown = __builtin_amdgcn_exp2f(a2 * sdt);
            float aq = aown;
            float hs = Hc[cl * kN + n];
            bq = fmaf(aq, hs * firstf, bq);
            scan16_up(bq, aq, hs);
            // forward, pass 2: the states; the output (for the gate's derivative) and dC
            float pC[kK];
            {
                float Cv[kK];
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) *(float4 *)&Cv[4 * pc] = *(const float4 *)&Cc[n * kFP + pc * (kLPR * 4)];
                float h = hs;
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    h = fmaf(e[j], h, u[j]);
                    hh[j] = h;
                    yv[j] = fmaf(Cv[j], h, yv[j]);
                    c[j] = Cv[j] * dyp[j];
                    pC[j] = dyp[j] * h;
                }
            }
            {
                float r4[4];
                rows4_sum(pC, r4);
                *(float4 *)&redC[16 * l + 4 * row] = make_float4(r4[0], r4[1], r4[2], r4[3]);
            }
            // reverse, pass 1: this lane's map of the adjoint, from a zero input
            float rb = 0.f;
#pragma unroll
            for (int j = kK - 1; j >= 0; --j) rb = e[j] * (c[j] + rb);
            float ra = aown;
            float gs = Gc[cl * kN + n];  // what the later chunk hands back, entering through lane 15
            rb = fmaf(ra, gs * lastf, rb);
            scan16_down(rb, ra, gs);
            if (l == 0) Gc[cl * kN + n] = rb;  // handed to the earlier chunk
            // reverse, pass 2: g_t and every derivative of the step
            float pB[kK];
            float dAl = 0.f;
            {
                float Bv[kK];
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) *(float4 *)&Bv[4 * pc] = *(const float4 *)&Bc[n * kFP + pc * (kLPR * 4)];
#pragma unroll
                for (int j = kK - 1; j >= 0; --j) {
                    const float gq = c[j] + gs;
                    const float gw = gq * (hh[j] - u[j]);
                    dAl = fmaf(dt[j], gw, dAl);
                    accdd[j] = fmaf(Araw, gw, accdd[j]);
                    acc1[j] = fmaf(gq, u[j], acc1[j]);
                    accx[j] = fmaf(gq, Bv[j], accx[j]);
                    pB[j] = gq * dlx[j];
                    gs = e[j] * gq;
                }
            }
            {
                float r4[4];
                rows4_sum(pB, r4);
                *(float4 *)&redB[16 * l + 4 * row] = make_float4(r4[0], r4[1], r4[2], r4[3]);
            }
            dAl = rowsum16(dAl);
            if (l == kLPR - 1) dAs[cl * kN + n] += dAl;
            lds_barrier();
            {
                // channel sums of this state's dB, dC for step tid of the chunk
                float sB = 0.f, sC = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    sB += red[w * kCH + tid];
                    sC += red[4 * kCH + w * kCH + tid];
                }
                if (s0 + tid < L) {
                    float *dst = p.wsBC + (((((int64_t)k * p.ntc + tc) * p.batch + b) * 2) * kN + n) * L + s0 + tid;
                    dst[0] = sB;
                    dst[(int64_t)kN * L] = sC;
                }
            }
            lds_barrier();
        }

        // ---- per (step, channel) derivatives: dx, ddelta, dz
        float o0[kK], o1[kK], o2[kK];
        float dbl = 0.f;
        {
            float df[kK], yf[kK], zf[kK];
            constexpr int V = S::kV;
            const T *tl[3] = {dtl, dyt, zt};
            float *fl[3] = {df, yf, zf};
#pragma unroll
            for (int m = 0; m < 3; ++m) {
#pragma unroll
                for (int pc = 0; pc < kK / V; ++pc) {
                    const uint4 v4 = *(const uint4 *)&tl[m][cl * S::kXP + pc * (kLPR * V) + l * V];
                    const uint32_t w4[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        if constexpr (sizeof(T) == 2)
                            fl[m][pc * V + i] = __uint_as_float(i & 1 ? w4[i >> 1] & 0xFFFF0000u : w4[i >> 1] << 16);
                        else
                            fl[m][pc * V + i] = __uint_as_float(w4[i]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kK; ++j) {
                float ddt = accdd[j] + (dt[j] != 0.f ? acc1[j] / dt[j] : 0.f);
                if (p.softplus) ddt *= sigmoidf_(df[j] + bias);
                ddt = j < lim ? ddt : 0.f;
                o0[j] = dt[j] * accx[j] + Dd * dyp[j];  // dx
                o1[j] = ddt;                            // d(delta)
                if constexpr (multi) {
                    o2[j] = yv[j];  // this direction's output; dz waits for the sum over directions
                } else if (z) {
                    const float sg = sigmoidf_(zf[j]);
                    o2[j] = yf[j] * yv[j] * sg * (1.f + zf[j] * (1.f - sg));
                } else {
                    o2[j] = 0.f;
                }
                dbl += ddt;
            }
        }
        dDl = rowsum16(dDl);
        dbl = rowsum16(dbl);
        if (l == kLPR - 1) {
            dDs[2 * cl] += dDl;
            dDs[2 * cl + 1] += dbl;
        }
        // out through the B and C tiles (free after the state loop): dx and ddelta, then dz
#pragma unroll
        for (int round = 0; round < 2; ++round) {
            if (round == 1 && !(z && p.dz)) break;
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
                const float *va = round == 0 ? o0 : o2;
                *(float4 *)&Bs[cl * kFP + pc * (kLPR * 4) + 4 * l] =
                    make_float4(va[4 * pc], va[4 * pc + 1], va[4 * pc + 2], va[4 * pc + 3]);
                if (round == 0)
                    *(float4 *)&Cs[cl * kFP + pc * (kLPR * 4) + 4 * l] =
                        make_float4(o1[4 * pc], o1[4 * pc + 1], o1[4 * pc + 2], o1[4 * pc + 3]);
            }
            lds_barrier();
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int sl = so + 128 * r;
                const int64_t s = s0 + sl;
                if (nv <= 0 || s >= L) continue;
                const int64_t off = (rowb + visit<KIND>(p, k, s)) * dim + cg;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = Bs[(8 * g + e) * kFP + fpos(sl)];
                if constexpr (multi) {
                    // add the earlier directions' sum; keep it, or finish dx / dz
                    float* acc = round == 0 ? p.wsX : p.wsY;
                    if (k > 0) {
                        float w8[8];
                        load_f8(acc + off, nv, vec, w8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] += w8[e];
                    }
                    if (!last) {
                        store8(acc + off, nv, vec, v);
                    } else if (round == 0) {
                        store8((T *)p.dx + off, nv, vec, v);
                    } else {
                        const int xs = S::xpos(sl);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float dyv = Io<T>::f32(dyt[(8 * g + e) * S::kXP + xs]);
                            const float zv = Io<T>::f32(zt[(8 * g + e) * S::kXP + xs]);
                            const float sg = sigmoidf_(zv);
                            v[e] = dyv * v[e] * sg * (1.f + zv * (1.f - sg));
                        }
                        store8((T *)p.dz + off, nv, vec, v);
                    }
                } else {
                    store8((T *)(round == 0 ? p.dx : p.dz) + off, nv, vec, v);
                }
                if (round == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = Cs[(8 * g + e) * kFP + fpos(sl)];
                    store8((T *)p.ddelta + k * tok + off, nv, vec, v);
                }
            }
            lds_barrier();
        }
    }
    lds_barrier();
    {
        const int ch = tid / kN, n = tid % kN;
        if (c0 + ch < dim) {
            if (p.dh0) p.dh0[((int64_t)b * dim + c0 + ch) * kN + n] = Gc[tid];
            p.wsA[(((int64_t)k * p.batch + b) * dim + c0 + ch) * kN + n] = dAs[tid];
        }
        if (tid < CT && c0 + tid < dim) {
            p.wsD[(((int64_t)k * p.batch + b) * dim + c0 + tid) * 2] = dDs[2 * tid];
            p.wsD[(((int64_t)k * p.batch + b) * dim + c0 + tid) * 2 + 1] = dDs[2 * tid + 1];
        }
    }
  }
}

struct BwdReduceParams {
    const float *wsBC, *wsA, *wsD;
    void *dB, *dC;
    float *dA, *dD, *dbias;
    int64_t L, dim;
    int H, Wd, win;  // scan order (dB, dC partials are by scan step)
    FastDiv dH, dWin, dWin2, dNx, dNy;
    int batch, ntc, ndir;
};

// dB[k,b,pi_k(t),:], dC[k,b,pi_k(t),:] = sum over the channel tiles of their partials for scan
// step t (one thread per (k, b, t)); dA, dD, ddelta_bias = sum over the batch rows (one thread
// per (k, channel, state)).
template <typename T, int KIND>
__global__ __launch_bounds__(256) void selscan_bwd_reduce(BwdReduceParams f) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nbt = (int64_t)f.ndir * f.batch * f.L;
    if (i < nbt) {
        const int64_t kb = i / f.L, t = i % f.L;  // kb = k * batch + b
        const int k = (int)(kb / f.batch), b = (int)(kb % f.batch);
        const int64_t row = kb * f.L + visit<KIND>(f, k, t);
#pragma unroll 1
        for (int qt = 0; qt < 2; ++qt) {
            float acc[kN];
#pragma unroll
            for (int n = 0; n < kN; ++n) acc[n] = 0.f;
#pragma unroll 1
            for (int c = 0; c < f.ntc; ++c) {
                const float *src = f.wsBC + ((((int64_t)k * f.ntc + c) * f.batch + b) * 2 + qt) * kN * f.L + t;
#pragma unroll
                for (int n = 0; n < kN; ++n) acc[n] += src[(int64_t)n * f.L];
            }
            T *dst = (T *)(qt == 0 ? f.dB : f.dC) + row * kN;
            store8(dst, 8, false, acc);
            store8(dst + 8, 8, false, acc + 8);
        }
        return;
    }
    const int64_t j = i - nbt, dn = f.dim * kN;
    if (j < f.ndir * dn) {
        const int64_t k = j / dn, jj = j % dn;
        float s = 0.f;
        for (int b = 0; b < f.batch; ++b) s += f.wsA[(k * f.batch + b) * dn + jj];
        f.dA[j] = s;
        if (jj % kN < 2) {
            const int64_t d = jj / kN;
            float t = 0.f;
            for (int b = 0; b < f.batch; ++b) t += f.wsD[((k * f.batch + b) * f.dim + d) * 2 + jj % kN];
            float *o = jj % kN == 0 ? f.dD : f.dbias;
            if (o) o[k * f.dim + d] = t;
        }
    }
}

// workspace of the backward: dB/dC tile partials, dA and dD/dbias batch-row partials, and
// with several directions the dx and pre-gate output sums
size_t bwd_ws_parts(int ndir, int64_t batch, int64_t L, int64_t dim, size_t part[5]) {
    const int64_t ntc = (dim + kTC - 1) / kTC;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t K = (size_t)ndir;
    part[0] = up(K * (size_t)ntc * (size_t)batch * 2 * kN * (size_t)L * 4);
    part[1] = up(K * (size_t)batch * (size_t)dim * kN * 4);
    part[2] = up(K * (size_t)batch * (size_t)dim * 2 * 4);
    part[3] = part[4] = ndir > 1 ? up((size_t)batch * (size_t)L * (size_t)dim * 4) : 0;
    return part[0] + part[1] + part[2] + part[3] + part[4];
}

struct BwdProblem {
    const void *x, *delta, *B, *C, *z, *dy;
    const float *A, *D, *bias, *ckpt;
    void *dx, *ddelta, *dB, *dC, *dz;
    float *dA, *dD, *dbias, *dh0;
    void *ws;
    int64_t batch, L, dim;
    int dtype;
    unsigned flags;
    int kind = SELSCAN_OP_FWD;
    int ndir = 1;
    int64_t H = 0, W = 0, win = 0;
};

int bwd_validate(const BwdProblem &p, int64_t dstate, size_t ws_bytes) {
    if (p.batch < 0 || p.L < 0 || p.dim < 0 || p.H < 0 || p.W < 0 || dstate < 0) return SELSCAN_E_SHAPE;
    if (p.dtype != SELSCAN_F32 && p.dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (p.flags & ~SELSCAN_FLAG_DELTA_SOFTPLUS) return SELSCAN_E_UNSUPPORTED;
    if (dstate != kN) return SELSCAN_E_UNSUPPORTED;
    if ((p.kind == SELSCAN_OP_SS2D || p.kind == SELSCAN_OP_LOCAL_SS2D) &&
        (p.L > 0x7FFFFFFF || p.H > 0x7FFFFFFF || p.W > 0x7FFFFFFF))
        return SELSCAN_E_UNSUPPORTED;
    if (p.kind == SELSCAN_OP_LOCAL_SS2D && (p.win < 1 || p.H % p.win || p.W % p.win)) return SELSCAN_E_SHAPE;
    if (p.batch == 0 || p.dim == 0) return SELSCAN_OK;
    if (!p.dA) return SELSCAN_E_NULL;
    if (p.L > 0 && (!p.x || !p.delta || !p.A || !p.B || !p.C || !p.ckpt || !p.dy || !p.dx || !p.ddelta ||
                    !p.dB || !p.dC))
        return SELSCAN_E_NULL;
    const size_t s = p.dtype == SELSCAN_BF16 ? 2 : 4;
    const void *io[] = {p.x, p.delta, p.B, p.C, p.z, p.dy, p.dx, p.ddelta, p.dB, p.dC, p.dz};
    for (const void *q : io)
        if (q && !aligned(q, s)) return SELSCAN_E_ALIGN;
    const void *f32[] = {p.A, p.D, p.bias, p.ckpt, p.dA, p.dD, p.dbias, p.dh0, p.ws};
    for (const void *q : f32)
        if (q && !aligned(q, 4)) return SELSCAN_E_ALIGN;
    size_t part[5];
    const size_t need = bwd_ws_parts(p.ndir, p.batch, p.L, p.dim, part);
    if (!p.ws || ws_bytes < need) return SELSCAN_E_WORKSPACE;
    const size_t K = (size_t)p.ndir;
    const size_t tok = (size_t)p.batch * p.L * p.dim * s, bc = (size_t)p.batch * p.L * kN * s;
    const size_t dn = (size_t)p.dim * kN * 4, dv = (size_t)p.dim * 4, hs = (size_t)p.batch * p.dim * kN * 4;
    const Span in[] = {{p.x, tok},        {p.delta, K * tok}, {p.B, K * bc},   {p.C, K * bc},
                       {p.z, tok},        {p.dy, tok},        {p.A, K * dn},   {p.D, K * dv},
                       {p.bias, K * dv},  {p.ckpt, K * ckpt_bytes_for(p.batch, p.L, p.dim)}};
    const Span out[] = {{p.dx, tok},       {p.ddelta, K * tok}, {p.dB, K * bc},    {p.dC, K * bc},
                        {p.z ? p.dz : nullptr, tok},            {p.dA, K * dn},    {p.dD, K * dv},
                        {p.dbias, K * dv}, {p.dh0, hs},         {p.ws, need}};
    constexpr int NO = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < NO; ++i) {
        for (const Span &q : in)
            if (overlap(out[i], q)) return SELSCAN_E_ALIAS;
        for (int j = i + 1; j < NO; ++j)
            if (overlap(out[i], out[j])) return SELSCAN_E_ALIAS;
    }
    return SELSCAN_OK;
}

template <typename T, int KIND>
int bwd_launch_kind(const BwdProblem &q, void *stream) {
    BwdParams a;
    a.x = q.x, a.delta = q.delta, a.B = q.B, a.C = q.C, a.z = q.z, a.dy = q.dy;
    a.A = q.A, a.D = q.D, a.bias = q.bias, a.ckpt = q.ckpt;
    a.dx = q.dx, a.ddelta = q.ddelta, a.dz = q.z ? q.dz : nullptr, a.dh0 = q.dh0;
    size_t part[5];
    bwd_ws_parts(q.ndir, q.batch, q.L, q.dim, part);
    char *w = (char *)q.ws;
    a.wsBC = (float *)w;
    a.wsA = (float *)(w + part[0]);
    a.wsD = (float *)(w + part[0] + part[1]);
    a.wsX = q.ndir > 1 ? (float *)(w + part[0] + part[1] + part[2]) : nullptr;
    a.wsY = q.ndir > 1 ? (float *)(w + part[0] + part[1] + part[2] + part[3]) : nullptr;
    a.dim = q.dim;
    set_order(a, q.kind, q.L, q.H, q.W, q.win);
    a.batch = (int)q.batch, a.ndir = q.ndir;
    a.softplus = (q.flags & SELSCAN_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
    a.ntc = (int)((q.dim + kTC - 1) / kTC);
    const void *rows[] = {q.x, q.delta, q.dy, q.z, q.dx, q.ddelta, q.dz, a.wsX, a.wsY};
    bool vec = q.dim % 8 == 0;
    for (const void *r : rows)
        if (r && !aligned(r, 16)) vec = false;
    a.vec = vec;
    a.vecbc = aligned(q.B, 16) && aligned(q.C, 16);
    const int64_t blocks = q.batch * (int64_t)a.ntc;
    if (blocks > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel((const void *)&selscan_bwd_chunked<T, KIND>, dim3((unsigned)blocks), dim3(256),
                                   args, 0, (hipStream_t)stream);
    if (e == hipSuccess) {
        BwdReduceParams f;
        f.wsBC = a.wsBC, f.wsA = a.wsA, f.wsD = a.wsD;
        f.dB = q.dB, f.dC = q.dC, f.dA = q.dA, f.dD = q.dD, f.dbias = q.dbias;
        f.dim = q.dim;
        set_order(f, q.kind, q.L, q.H, q.W, q.win);
        f.batch = (int)q.batch, f.ntc = a.ntc, f.ndir = q.ndir;
        const int64_t items = q.ndir * (q.batch * q.L + q.dim * kN);
        const int64_t rb = (items + 255) / 256;
        if (rb > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
        void *fargs[] = {&f};
        e = hipLaunchKernel((const void *)&selscan_bwd_reduce<T, KIND>, dim3((unsigned)rb), dim3(256), fargs, 0,
                            (hipStream_t)stream);
    }
    if (e != hipSuccess) {
        strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
        return SELSCAN_E_HIP;
    }
    return SELSCAN_OK;
}

template <typename T>
int bwd_launch(const BwdProblem &q, void *stream) {
    if (q.kind == SELSCAN_OP_FWD) return bwd_launch_kind<T, SELSCAN_OP_FWD>(q, stream);
    if (q.kind == SELSCAN_OP_BIDIR) return bwd_launch_kind<T, SELSCAN_OP_BIDIR>(q, stream);
    if (q.kind == SELSCAN_OP_SS2D) return bwd_launch_kind<T, SELSCAN_OP_SS2D>(q, stream);
    return bwd_launch_kind<T, SELSCAN_OP_LOCAL_SS2D>(q, stream);
}

int bwd_run(BwdProblem &p, int64_t dstate, size_t ws_bytes, void *stream) {
    const int rc = bwd_validate(p, dstate, ws_bytes);
    if (rc != SELSCAN_OK) return rc;
    if (p.batch == 0 || p.dim == 0) return SELSCAN_OK;
    if (p.batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    if (p.dtype == SELSCAN_BF16) return bwd_launch<uint16_t>(p, stream);
    return bwd_launch<float>(p, stream);
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

}  // namespace

extern "C" {

int selscan_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
                const void *z, const float *delta_bias, unsigned flags, void *y, int64_t batch, int64_t seqlen,
                int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p{x, delta, B, C, z, A, D, delta_bias, y, workspace, batch, seqlen, dim, 0, 0, 1, SELSCAN_OP_FWD,
              io_dtype, flags};
    return run(p, dstate, workspace_bytes, stream);
}

int selscan_fwd_state(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                      const float *h0, float *h_last, float *chunk_states, int64_t batch, int64_t seqlen,
                      int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes,
                      void *stream) {
    Problem p{x, delta, B, C, z, A, D, delta_bias, y, workspace, batch, seqlen, dim, 0, 0, 1, SELSCAN_OP_FWD,
              io_dtype, flags, h0, h_last, chunk_states};
    return run(p, dstate, workspace_bytes, stream);
}

int selscan_bidir_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                      int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                      size_t workspace_bytes, void *stream) {
    Problem p{x, delta, B, C, z, A, D, delta_bias, y, workspace, batch, seqlen, dim, 0, 0, 2, SELSCAN_OP_BIDIR,
              io_dtype, flags};
    return run(p, dstate, workspace_bytes, stream);
}

int ss2d_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
             const void *z, const float *delta_bias, unsigned flags, void *y, int64_t batch, int64_t H, int64_t W,
             int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (H < 0 || W < 0) return SELSCAN_E_SHAPE;
    Problem p{x, delta, B, C, z, A, D, delta_bias, y, workspace, batch, H * W, dim, H, W, 4, SELSCAN_OP_SS2D,
              io_dtype, flags};
    return run(p, dstate, workspace_bytes, stream);
}

int local_ss2d_fwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
                   const void *z, const float *delta_bias, unsigned flags, void *y, int64_t batch, int64_t H,
                   int64_t W, int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                   size_t workspace_bytes, void *stream) {
    if (H < 0 || W < 0) return SELSCAN_E_SHAPE;
    Problem p{x, delta, B, C, z, A, D, delta_bias, y, workspace, batch, H * W, dim, H, W, 4, SELSCAN_OP_LOCAL_SS2D,
              io_dtype, flags};
    p.win = window;
    return run(p, dstate, workspace_bytes, stream);
}

size_t selscan_workspace_bytes(int op, int64_t batch, int64_t seqlen_or_hw, int64_t dim, int64_t dstate,
                               int io_dtype) {
    (void)dstate;
    (void)io_dtype;
    if (batch <= 0 || seqlen_or_hw <= 0 || dim <= 0) return 0;
    if (op != SELSCAN_OP_FWD && op != SELSCAN_OP_BIDIR && op != SELSCAN_OP_SS2D && op != SELSCAN_OP_LOCAL_SS2D)
        return 0;
    return workspace_bytes_for(op, batch, seqlen_or_hw, dim);
}

size_t selscan_chunk_states_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
    if (batch <= 0 || seqlen <= 0 || dim <= 0 || dstate != kN) return 0;
    return ckpt_bytes_for(batch, seqlen, dim);
}

size_t selscan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype) {
    (void)io_dtype;
    if (batch <= 0 || seqlen < 0 || dim <= 0 || dstate != kN) return 0;
    size_t part[5];
    return bwd_ws_parts(1, batch, seqlen, dim, part);
}

int selscan_bwd(const void *x, const void *delta, const float *A, const void *B, const void *C, const float *D,
                const void *z, const float *delta_bias, unsigned flags, const float *chunk_states, const void *dy,
                void *dx, void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz, float *ddelta_bias,
                float *dh0, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                void *workspace, size_t workspace_bytes, void *stream) {
    BwdProblem p{x,  delta, B,  C,  z,     dy,    A,     D,     delta_bias, chunk_states, dx,    ddelta,
                 dB, dC,    dz, dA, dD,    ddelta_bias, dh0, workspace,  batch,        seqlen, dim,
                 io_dtype, flags};
    return bwd_run(p, dstate, workspace_bytes, stream);
}

int selscan_scan_fwd(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                     const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                     float *chunk_states, int64_t batch, int64_t seqlen, int64_t H, int64_t W, int64_t window,
                     int64_t dim, int64_t dstate, int io_dtype, void *workspace, size_t workspace_bytes,
                     void *stream) {
    int64_t L;
    int ndir;
    const int rc = resolve_op(op, seqlen, H, W, &L, &ndir);
    if (rc != SELSCAN_OK) return rc;
    const bool two_d = op == SELSCAN_OP_SS2D || op == SELSCAN_OP_LOCAL_SS2D;
    Problem p{x,     delta, B, C, z, A, D, delta_bias, y, workspace, batch, L, dim, two_d ? H : 0, two_d ? W : 0,
              ndir,  op,    io_dtype, flags};
    p.ckpt = chunk_states;
    p.win = op == SELSCAN_OP_LOCAL_SS2D ? window : 0;
    return run(p, dstate, workspace_bytes, stream);
}

int selscan_scan_bwd(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                     const float *D, const void *z, const float *delta_bias, unsigned flags,
                     const float *chunk_states, const void *dy, void *dx, void *ddelta, float *dA, void *dB,
                     void *dC, float *dD, void *dz, float *ddelta_bias, int64_t batch, int64_t seqlen, int64_t H,
                     int64_t W, int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                     size_t workspace_bytes, void *stream) {
    int64_t L;
    int ndir;
    const int rc = resolve_op(op, seqlen, H, W, &L, &ndir);
    if (rc != SELSCAN_OK) return rc;
    const bool two_d = op == SELSCAN_OP_SS2D || op == SELSCAN_OP_LOCAL_SS2D;
    BwdProblem p{x,  delta, B,  C,  z,     dy,    A,     D,     delta_bias, chunk_states, dx,    ddelta,
                 dB, dC,    dz, dA, dD,    ddelta_bias, nullptr, workspace, batch,      L,      dim,
                 io_dtype, flags};
    p.kind = op, p.ndir = ndir;
    p.H = two_d ? H : 0, p.W = two_d ? W : 0;
    p.win = op == SELSCAN_OP_LOCAL_SS2D ? window : 0;
    return bwd_run(p, dstate, workspace_bytes, stream);
}

size_t selscan_scan_chunk_states_bytes(int op, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
    const int ndir = ndir_of(op);
    if (ndir == 0 || batch <= 0 || seqlen <= 0 || dim <= 0 || dstate != kN) return 0;
    return (size_t)ndir * ckpt_bytes_for(batch, seqlen, dim);
}

size_t selscan_scan_bwd_workspace_bytes(int op, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                        int io_dtype) {
    (void)io_dtype;
    const int ndir = ndir_of(op);
    if (ndir == 0 || batch <= 0 || seqlen < 0 || dim <= 0 || dstate != kN) return 0;
    size_t part[5];
    return bwd_ws_parts(ndir, batch, seqlen, dim, part);
}

const char *selscan_status_str(int status) {
    switch (status) {
        case SELSCAN_OK: return "ok";
        case SELSCAN_E_NULL: return "a required pointer is NULL";
        case SELSCAN_E_SHAPE: return "a size is negative";
        case SELSCAN_E_ALIGN: return "a pointer is not aligned to its element size";
        case SELSCAN_E_ALIAS: return "the output overlaps an input or the workspace";
        case SELSCAN_E_UNSUPPORTED: return "unsupported dstate, dtype, flag or size";
        case SELSCAN_E_WORKSPACE: return "workspace missing or too small";
        case SELSCAN_E_HIP: return "the HIP runtime rejected the kernel launch";
        default: return "unknown status";
    }
}

int selscan_abi_version(void) { return SELSCAN_ABI_VERSION; }

const char *selscan_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
