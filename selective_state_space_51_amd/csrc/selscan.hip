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

constexpr int kN = 16;                   // d_state supported by this version
constexpr int kK = 16;                   // consecutive scan steps per lane
constexpr int kLanesPerRow = 16;         // lanes sharing one channel (one DPP row)
constexpr int kRows = 4;                 // channels per wave
constexpr int kWaves = 4;                // waves per workgroup
constexpr int kThreads = 64 * kWaves;    // 256
constexpr int kCT = kRows * kWaves;      // channels per workgroup tile (16)
constexpr int kCH = kLanesPerRow * kK;   // scan steps per chunk (256)
constexpr int kSegF = kK + 4;            // fp32 LDS stride of one lane segment (floats)
constexpr int kColF = kLanesPerRow * kSegF + 4;  // fp32 LDS column pitch (floats)
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kCH == kThreads, "B/C staging maps one chunk row to one thread");
static_assert(kCT % 4 == 0, "channel groups of 4");

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
};

size_t workspace_bytes_for(int op, int64_t batch, int64_t L, int64_t dim) {
    if (op == SELSCAN_OP_FWD) return 0;
    return (size_t)batch * (size_t)L * (size_t)dim * sizeof(float);
}

int validate(const Problem &p, int64_t dstate, size_t ws_bytes) {
    if (p.batch < 0 || p.L < 0 || p.dim < 0 || p.H < 0 || p.W < 0 || dstate < 0) return SELSCAN_E_SHAPE;
    if (p.dtype != SELSCAN_F32 && p.dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (p.flags & ~SELSCAN_FLAG_DELTA_SOFTPLUS) return SELSCAN_E_UNSUPPORTED;
    if (dstate != kN) return SELSCAN_E_UNSUPPORTED;
    if (p.batch == 0 || p.L == 0 || p.dim == 0) return SELSCAN_OK;
    if (!p.x || !p.delta || !p.A || !p.B || !p.C || !p.y) return SELSCAN_E_NULL;
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
    return SELSCAN_OK;
}

// ------------------------------------------------------------------------------------
// device side
// ------------------------------------------------------------------------------------

struct Params {
    const void *x, *delta, *B, *C, *z;
    const float *A, *D, *bias;
    void *y;
    float *ws;        // fp32 [batch][L][dim] partial sums when ndir > 1
    int64_t L, dim, H;
    int batch, ndir, kind, softplus;
    int vec;          // rows of 4 channels may be moved as one vector
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
    // round to nearest even; a NaN stays a (quiet) NaN
    __device__ static uint16_t to(float v) {
        const uint32_t u = __float_as_uint(v);
        const uint32_t r =
            (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
        return (uint16_t)r;
    }
};

// io-dtype column tile geometry: [channel][segment-padded steps]
template <typename T>
struct Tile {
    static constexpr int kSegE = kK + Io<T>::kPadE;
    static constexpr int kColE = kLanesPerRow * kSegE + Io<T>::kPadE;
    static constexpr int kBytes = kCT * kColE * (int)sizeof(T);
    static constexpr int kYBytes = kCT * kColF * 4;
    static constexpr int kXDBytes = 2 * kBytes > kYBytes ? 2 * kBytes : kYBytes;  // x, delta or y
    static constexpr int kBCBytes = 2 * kN * kColF * 4;
    static constexpr int kSmem = kXDBytes + kBCBytes;
    __device__ static int seg(int i) { return (i / kK) * kSegE + (i % kK); }
};
__device__ __forceinline__ int segf(int i) { return (i / kK) * kSegF + (i % kK); }

// row (token or pixel) visited at scan step l by direction k
__device__ __forceinline__ int64_t visit(int kind, int k, int64_t l, int64_t L, int64_t H) {
    if (kind == SELSCAN_OP_FWD) return l;
    if (kind == SELSCAN_OP_BIDIR) return k == 0 ? l : L - 1 - l;
    if (k >= 2) l = L - 1 - l;
    if (k == 0 || k == 2) return l;
    return (l % H) * (L / H) + l / H;
}

// softplus(w) = log(1 + e^w) without overflow
__device__ __forceinline__ float softplus(float w) { return w > 0.f ? w + log1pf(__expf(-w)) : log1pf(__expf(w)); }

// silu(z) = z * sigmoid(z) on v_exp_f32 and v_rcp_f32 (large |z| saturates to 0 or z)
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// DPP move within 16-lane rows; lanes whose source is outside the row get `old`
template <int CTRL>
__device__ __forceinline__ float dpp(float old, float src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                  __builtin_bit_cast(int, src), CTRL, 0xF, 0xF,
                                                                  false));
}
constexpr int kRowShr = 0x110;  // row_shr:n = kRowShr + n
constexpr int kRowRor1 = 0x121;  // row_ror:1

// 4 consecutive io elements of one row -> float[4]; elements past `n` read as 0
template <typename T>
__device__ __forceinline__ void load4(const T *p, int n, bool vec, float v[4]) {
    if (vec && n >= 4) {
        if constexpr (sizeof(T) == 4) {
            const float4 q = *(const float4 *)p;
            v[0] = q.x, v[1] = q.y, v[2] = q.z, v[3] = q.w;
        } else {
            const uint2 q = *(const uint2 *)p;
            v[0] = __uint_as_float(q.x << 16), v[1] = __uint_as_float(q.x & 0xFFFF0000u);
            v[2] = __uint_as_float(q.y << 16), v[3] = __uint_as_float(q.y & 0xFFFF0000u);
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e < n ? Io<T>::f32(p[e]) : 0.f;
}

template <typename T>
__device__ __forceinline__ void store4(T *p, int n, bool vec, const float v[4]) {
    if (vec && n >= 4) {
        if constexpr (sizeof(T) == 4) {
            *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
        } else {
            uint2 q;
            q.x = (uint32_t)Io<T>::to(v[0]) | ((uint32_t)Io<T>::to(v[1]) << 16);
            q.y = (uint32_t)Io<T>::to(v[2]) | ((uint32_t)Io<T>::to(v[3]) << 16);
            *(uint2 *)p = q;
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < n) p[e] = Io<T>::to(v[e]);
}

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void selscan_chunked(Params p) {
    using TL = Tile<T>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[TL::kSmem];
    T *xt = (T *)smem;                       // x column tile [kCT][kColE]
    T *dtile = (T *)(smem + TL::kBytes);     // delta column tile
    float *yt = (float *)smem;               // y partial [kCT][kColF] (reuses x/delta space)
    float *Bs = (float *)(smem + TL::kXDBytes);  // [kN][kColF]
    float *Cs = Bs + kN * kColF;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, row = lane >> 4, l = lane & 15;
    // consecutive channel tiles on one XCD: workgroups are dealt round-robin over 8 XCDs
    const int G = gridDim.x, bi = blockIdx.x, q8 = G >> 3;
    const int tile = bi < (q8 << 3) ? (bi & 7) * q8 + (bi >> 3) : bi;
    const int b = tile / p.ntc;
    const int64_t c0 = (int64_t)(tile % p.ntc) * kCT;
    const int cl = wave * kRows + row;
    const int64_t c = c0 + cl;
    const bool cvalid = c < p.dim;
    const int64_t L = p.L, dim = p.dim;
    const int64_t tok = (int64_t)p.batch * L * dim, bcn = (int64_t)p.batch * L * kN;
    const int ncols = (int)(dim - c0 < kCT ? dim - c0 : kCT);  // valid channels in this tile
    const int nchunks = (int)((L + kCH - 1) / kCH);
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x;
    const T *z = (const T *)p.z;
    T *y = (T *)p.y;

    for (int k = 0; k < p.ndir; ++k) {
        const T *dl = (const T *)p.delta + k * tok;
        const T *Bk = (const T *)p.B + k * bcn;
        const T *Ck = (const T *)p.C + k * bcn;
        const int64_t cc = cvalid ? c : 0;
        float A2[kN], carry[kN];
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            A2[n] = p.A[(k * dim + cc) * kN + n] * kLog2e;
            carry[n] = 0.f;
        }
        const float Dd = p.D ? p.D[k * dim + cc] : 0.f;
        const float bias = p.bias ? p.bias[k * dim + cc] : 0.f;

        for (int q = 0; q < nchunks; ++q) {
            const int64_t s0 = (int64_t)q * kCH;
            __syncthreads();  // the previous chunk is done with every tile
            // ---- stage x and delta: rows of 4 channels, written column-major
#pragma unroll
            for (int m = 0; m < kCH * (kCT / 4) / kThreads; ++m) {
                const int item = tid + m * kThreads, i = item >> 2, g = item & 3;
                const int64_t s = s0 + i;
                float xv[4] = {0.f, 0.f, 0.f, 0.f}, dv[4] = {0.f, 0.f, 0.f, 0.f};
                const int nv = ncols - 4 * g;
                if (s < L && nv > 0) {
                    const int64_t off = ((int64_t)b * L + visit(p.kind, k, s, L, p.H)) * dim + c0 + 4 * g;
                    load4(x + off, nv, vec, xv);
                    load4(dl + off, nv, vec, dv);
                }
                const int si = TL::seg(i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (sizeof(T) == 4) {
                        xt[(4 * g + e) * TL::kColE + si] = xv[e];
                        dtile[(4 * g + e) * TL::kColE + si] = dv[e];
                    } else {
                        xt[(4 * g + e) * TL::kColE + si] = (T)(__float_as_uint(xv[e]) >> 16);
                        dtile[(4 * g + e) * TL::kColE + si] = (T)(__float_as_uint(dv[e]) >> 16);
                    }
                }
            }
            // ---- stage B and C for this chunk as fp32 [state][step]
            {
                const int i = tid;
                const int64_t s = s0 + i;
                float bv[kN], cv[kN];
                if (s < L) {
                    const int64_t roff = ((int64_t)b * L + visit(p.kind, k, s, L, p.H)) * kN;
                    if (p.vecbc) {
#pragma unroll
                        for (int h = 0; h < kN; h += 4) {
                            load4(Bk + roff + h, 4, true, bv + h);
                            load4(Ck + roff + h, 4, true, cv + h);
                        }
                    } else {
#pragma unroll
                        for (int n = 0; n < kN; ++n) {
                            bv[n] = Io<T>::f32(Bk[roff + n]);
                            cv[n] = Io<T>::f32(Ck[roff + n]);
                        }
                    }
                } else {
#pragma unroll
                    for (int n = 0; n < kN; ++n) bv[n] = cv[n] = 0.f;
                }
                const int sf = segf(i);
#pragma unroll
                for (int n = 0; n < kN; ++n) {
                    Bs[n * kColF + sf] = bv[n];
                    Cs[n * kColF + sf] = cv[n];
                }
            }
            __syncthreads();

            // ---- this lane's 16 steps of its channel
            float dt[kK], dx[kK], yv[kK];
            float sdt = 0.f;
            {
                const T *xc = xt + cl * TL::kColE + l * TL::kSegE;
                const T *dc = dtile + cl * TL::kColE + l * TL::kSegE;
                T xr[kK], dr[kK];
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    xr[j] = xc[j];
                    dr[j] = dc[j];
                }
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    const bool v = cvalid && (s0 + l * kK + j < L);
                    float d = Io<T>::f32(dr[j]) + bias;
                    if (p.softplus) d = softplus(d);
                    d = v ? d : 0.f;
                    const float xv = Io<T>::f32(xr[j]);
                    dt[j] = d;
                    dx[j] = d * xv;
                    yv[j] = Dd * xv;
                    sdt += d;
                }
            }
            const float *Bc = Bs + l * kSegF;
            const float *Cc = Cs + l * kSegF;
#pragma unroll
            for (int n = 0; n < kN; ++n) {
                const float a2 = A2[n];
                float e[kK], u[kK];
                float bb = 0.f;
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    e[j] = __builtin_amdgcn_exp2f(dt[j] * a2);
                    u[j] = dx[j] * Bc[n * kColF + j];
                    bb = fmaf(e[j], bb, u[j]);
                }
                float a = __builtin_amdgcn_exp2f(a2 * sdt);
                bb = fmaf(a, l == 0 ? carry[n] : 0.f, bb);
                // inclusive scan of the lanes' affine maps along the row
                {
                    float ap = dpp<kRowShr + 1>(1.f, a), bp = dpp<kRowShr + 1>(0.f, bb);
                    bb = fmaf(a, bp, bb);
                    a *= ap;
                    ap = dpp<kRowShr + 2>(1.f, a), bp = dpp<kRowShr + 2>(0.f, bb);
                    bb = fmaf(a, bp, bb);
                    a *= ap;
                    ap = dpp<kRowShr + 4>(1.f, a), bp = dpp<kRowShr + 4>(0.f, bb);
                    bb = fmaf(a, bp, bb);
                    a *= ap;
                    bp = dpp<kRowShr + 8>(0.f, bb);
                    bb = fmaf(a, bp, bb);
                }
                // lane l >= 1 starts from lane l-1's end state; lane 0 from the chunk carry;
                // lane 0 receives lane 15's end state, the carry of the next chunk
                const float rot = dpp<kRowRor1>(0.f, bb);
                float h = l == 0 ? carry[n] : rot;
                carry[n] = rot;
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    h = fmaf(e[j], h, u[j]);
                    yv[j] = fmaf(Cc[n * kColF + j], h, yv[j]);
                }
            }
            __syncthreads();  // x/delta tiles fully read before y reuses their space
            {
                float *yc = yt + cl * kColF + l * kSegF;
#pragma unroll
                for (int j = 0; j < kK; ++j) yc[j] = yv[j];
            }
            __syncthreads();
            // ---- leave: add earlier directions, gate, store y (or keep the partial sum)
#pragma unroll
            for (int m = 0; m < kCH * (kCT / 4) / kThreads; ++m) {
                const int item = tid + m * kThreads, i = item >> 2, g = item & 3;
                const int64_t s = s0 + i;
                const int nv = ncols - 4 * g;
                if (s >= L || nv <= 0) continue;
                const int64_t off = ((int64_t)b * L + visit(p.kind, k, s, L, p.H)) * dim + c0 + 4 * g;
                float v[4];
                const int sf = segf(i);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = yt[(4 * g + e) * kColF + sf];
                if (k > 0) {
                    float w4[4];
                    load4(p.ws + off, nv, vec, w4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += w4[e];
                }
                if (k == p.ndir - 1) {
                    if (z) {
                        float zv[4];
                        load4(z + off, nv, vec, zv);
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] *= silu(zv[e]);
                    }
                    store4(y + off, nv, vec, v);
                } else {
                    store4(p.ws + off, nv, vec, v);
                }
            }
        }
    }
}

int launch(const Problem &p, void *stream) {
    const size_t s = p.dtype == SELSCAN_BF16 ? 2 : 4;
    Params a;
    a.x = p.x, a.delta = p.delta, a.B = p.B, a.C = p.C, a.z = p.z;
    a.A = p.A, a.D = p.D, a.bias = p.bias, a.y = p.y;
    a.ws = p.ndir > 1 ? (float *)p.ws : nullptr;
    a.L = p.L, a.dim = p.dim, a.H = p.H;
    a.batch = (int)p.batch, a.ndir = p.ndir, a.kind = p.kind;
    a.softplus = (p.flags & SELSCAN_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
    const void *rows[] = {p.x, p.delta, p.z, p.y};
    bool vec = p.dim % 4 == 0 && (!a.ws || aligned(a.ws, 16));
    for (const void *q : rows)
        if (q && !aligned(q, 4 * s)) vec = false;
    a.vec = vec;
    a.vecbc = aligned(p.B, 16) && aligned(p.C, 16);
    a.ntc = (int)((p.dim + kCT - 1) / kCT);
    const int64_t blocks = p.batch * (int64_t)a.ntc;
    if (blocks > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    void *args[] = {&a};
    const void *fn = p.dtype == SELSCAN_BF16 ? (const void *)&selscan_chunked<uint16_t>
                                             : (const void *)&selscan_chunked<float>;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kThreads), args, 0, (hipStream_t)stream);
    if (e != hipSuccess) {
        strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
        return SELSCAN_E_HIP;
    }
    return SELSCAN_OK;
}

int run(Problem &p, int64_t dstate, size_t ws_bytes, void *stream) {
    int rc = validate(p, dstate, ws_bytes);
    if (rc != SELSCAN_OK) return rc;
    if (p.batch == 0 || p.L == 0 || p.dim == 0) return SELSCAN_OK;
    if (p.batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    return launch(p, stream);
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

size_t selscan_workspace_bytes(int op, int64_t batch, int64_t seqlen_or_hw, int64_t dim, int64_t dstate,
                               int io_dtype) {
    (void)dstate;
    (void)io_dtype;
    if (batch <= 0 || seqlen_or_hw <= 0 || dim <= 0) return 0;
    if (op != SELSCAN_OP_FWD && op != SELSCAN_OP_BIDIR && op != SELSCAN_OP_SS2D) return 0;
    return workspace_bytes_for(op, batch, seqlen_or_hw, dim);
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
