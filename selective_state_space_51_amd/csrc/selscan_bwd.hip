// libselscan - backward of the selective scan (every scan order) for MI355X (gfx950),
// behind the C ABI declared in include/selscan.h.
#include "selscan_common.h"

namespace {

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
// with e_t h_{t-1} kept from the recomputed forward and sum_n g_t B_t x_t = x_t sum_n g_t B_t,
// the sum dx needs as well (one accumulator serves both).  dB and dC are summed over the
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
    int split;  // one direction per workgroup; dx and output partial rows per direction
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
    static constexpr int kRed = kDD + kTC * 8;              // channel sums of dB, dC: fp32 [2][4 waves][256]
    static constexpr int kBytes = kRed + 2 * 4 * kCH * 4;
    static_assert(kTC * kFP * 4 <= 2 * kIo, "an fp32 output tile fits in the x and delta tiles");
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

#ifdef SELSCAN_PHASE_CLOCKS
// per-wave phase clocks of the backward (diagnostic library only): 0 staging (loads and their
// commit to LDS), 1 prologue, 2 state loop outside its barriers, 3 and 4 the waits at its two
// barriers, 5 output
__device__ unsigned long long g_bwd_phase[kPhaseWaves * 8];
#endif

__device__ __forceinline__ float sigmoidf_(float w) { return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-w * kLog2e)); }

template <typename T, int KIND, bool ZOH>
// two workgroups per CU with bf16 io; the fp32 io tiles leave LDS for one
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void selscan_bwd_chunked(BwdParams p) {
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
    float *Os = (float *)(smem + S::kX);  // third output tile (x and delta space)

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l = lane & 15, row = lane >> 4;
    PhaseClock clk;
    const int cl = wave * 4 + row;
    const float firstf = l == 0 ? 1.f : 0.f, lastf = l == kLPR - 1 ? 1.f : 0.f;
    const int G = gridDim.x, bi = blockIdx.x, q8 = G >> 3;
    const int tile_all = bi < (q8 << 3) ? (bi & 7) * q8 + (bi >> 3) : bi;
    const int ntiles = p.batch * p.ntc;
    const bool split = multi && p.split;  // grid = directions x tiles
    const int tile = split ? tile_all % ntiles : tile_all;
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
  const int k_begin = split ? tile_all / ntiles : 0, k_end = split ? k_begin + 1 : ndir;
  for (int k = k_begin; k < k_end; ++k) {
    const T *dl = (const T *)p.delta + k * tok;
    const T *Bg = (const T *)p.B + k * bcn;
    const T *Cg = (const T *)p.C + k * bcn;
    const bool last = k == ndir - 1 && !split;
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

    // global -> registers for chunk q: x, delta, dy, z rows of steps 2p, 2p+1 (8 channels each),
    // the B and C rows of one step, the chunk's entry state.  Issued at the top of the chunk,
    // not a chunk ahead: the state loop holds every register, and keeping the loads' registers
    // live from the previous chunk's output phase into this one pushes the spill from 20 to over
    // 200 bytes per lane (measured slower).
    Raw8<T> r0[4], r1[4];
    uint32_t pbc[2][NW];
    float hck;
    auto fetch = [&](int q) {
        const int64_t s0 = (int64_t)q * kCH;
        const int64_t sa = s0 + 2 * pp, sbb = sa + 1;
        const T *src[4] = {x, dl, dy, z};
        // The lane's channel offset, made opaque per call: otherwise the compiler hoists one
        // 64-bit per-lane pointer per tensor out of the chunk loop, spills them across the state
        // loop, and reloads each right before its row load -- and waiting for a scratch reload
        // waits for every load issued before it, which serialises the staging loads.
        int64_t cgl = cg;
        asm volatile("" : "+v"(cgl));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            r0[m] = r1[m] = Raw8<T>{};
            if (!src[m]) continue;
            if (nv > 0 && sa < L) r0[m] = load_raw8(src[m] + ((rowb + visit<KIND>(p, k, sa)) * dim + cgl), nv, vec);
            if (nv > 0 && sbb < L) r1[m] = load_raw8(src[m] + ((rowb + visit<KIND>(p, k, sbb)) * dim + cgl), nv, vec);
        }
#pragma unroll
        for (int h = 0; h < NW; ++h) pbc[0][h] = pbc[1][h] = 0u;
        int sbl = sb;  // opaque per call, as cgl above
        asm volatile("" : "+v"(sbl));
        const int64_t s = s0 + sbl;
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
        int64_t own = (c0 + tid / kN) * kN + tid % kN;  // this thread's (channel, state) entry
        asm volatile("" : "+v"(own));
        hck = c0 + tid / kN < dim ? p.ckpt[(((int64_t)k * p.batch + b) * nchunks + q) * dim * kN + own] : 0.f;
    };
    auto commit = [&]() {
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
        Hc[tid] = hck;
    };
    clk.mark();
    for (int q = nchunks - 1; q >= 0; --q) {
        const int64_t s0 = (int64_t)q * kCH;
        // priority: staging, prologue and output above the state loop, whose priority alternates
        // with the chunk's parity so the two workgroups sharing a SIMD take turns ahead
        __builtin_amdgcn_s_setprio(2);
        fetch(q);
        lds_barrier();  // the previous (later) chunk is done with every tile
        commit();
        lds_barrier();
        clk.add(0);

        // ---- this lane's 16 steps of its channel
        const int64_t rem = L - (s0 + l * kK);
        const int lim = !cvalid ? 0 : (rem <= 0 ? 0 : (rem >= kK ? kK : (int)rem));
        // px: the step's input factor, delta x (Euler) or x (zero-order hold, whose input
        // coefficient differs per state)
        float dt[kK], px[kK], dyp[kK], yv[kK];
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
#pragma unroll
            for (int j = 0; j < kK; ++j) {
                const float w = df[j] + bias;
                dt[j] = p.softplus ? softplus(w) : w;
            }
            if (lim < kK) {
                // steps past the sequence end and channels past dim: delta = 0, the identity
                // step (lanes of full chunks skip this)
                const float limf = (float)lim;
#pragma unroll
                for (int j = 0; j < kK; ++j) dt[j] *= __builtin_amdgcn_fmed3f(limf - (float)j, 0.f, 1.f);
            }
#pragma unroll
            for (int j = 0; j < kK; ++j) {
                px[j] = ZOH ? xf[j] : dt[j] * xf[j];
                dyp[j] = z ? yf[j] * silu(zf[j]) : yf[j];
                yv[j] = Dd * xf[j];
                dDl = fmaf(dyp[j], xf[j], dDl);
                sdt += dt[j];
            }
        }
        // Euler: sum_n g A e h_{t-1};  sum_n g B  (d delta = accdd + x accx, dx = delta accx)
        // ZOH:   sum_n g A e h_{t-1} + x sum_n g e B;  sum_n g phi B  (d delta = accdd, dx = delta accx)
        float accdd[kK], accx[kK];
#pragma unroll
        for (int j = 0; j < kK; ++j) accdd[j] = accx[j] = 0.f;
        const float *Bc = Bs + 4 * l;
        const float *Cc = Cs + 4 * l;
        float *redB = red + wave * kCH, *redC = red + 4 * kCH + wave * kCH;
        // lane (row, l) holds the channel sums of steps 16 l + 4 row + (0..3); row r's slots are
        // rotated by 2 r, so that each 8-lane group of the float4 stores here, and each 32-lane
        // half of the step-ordered reads after the barrier, meets 32 distinct LDS banks
        const int rslot = 64 * row + 4 * ((l + 2 * row) & 15);
        const int rtid = 64 * ((tid >> 2) & 3) + 4 * (((tid >> 4) + 2 * ((tid >> 2) & 3)) & 15) + (tid & 3);

        if (q & 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        clk.add(1);
#pragma unroll 1
        for (int n = 0; n < kN; ++n) {
            const float a2 = As[cl * kN + n];
            const float Araw = a2 * kLn2;
            float e[kK], u[kK], eh[kK], c[kK];
            // forward, pass 1: from a zero state
            float bq;
            {
                float Bv[kK];
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) *(float4 *)&Bv[4 * pc] = *(const float4 *)&Bc[n * kFP + pc * (kLPR * 4)];
#pragma unroll
                for (int j = 0; j < kK; ++j) {
                    const float t = dt[j] * a2;
                    e[j] = __builtin_amdgcn_exp2f(t);
                    if constexpr (ZOH)
                        u[j] = dt[j] * px[j] * (zoh_phi(e[j], t) * Bv[j]);
                    else
                        u[j] = px[j] * Bv[j];
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
                    eh[j] = e[j] * h;  // e_t h_{t-1}
                    h = eh[j] + u[j];
                    yv[j] = fmaf(Cv[j], h, yv[j]);
                    c[j] = Cv[j] * dyp[j];
                    pC[j] = dyp[j] * h;
                }
            }
            {
                float r4[4];
                rows4_sum(pC, r4);
                *(float4 *)&redC[rslot] = make_float4(r4[0], r4[1], r4[2], r4[3]);
            }
            // reverse, pass 1: this lane's map of the adjoint, from a zero input.  Down the lane
            // g_j = c_j + e_{j+1} g_{j+1} (one FMA a step); the lane hands e_0 g_0 to its left
            // neighbour, and its multiplier is the product of its 16 decays, aown.
            float rg = c[kK - 1];
#pragma unroll
            for (int j = kK - 2; j >= 0; --j) rg = fmaf(e[j + 1], rg, c[j]);
            float rb = e[0] * rg;
            float ra = aown;
            float gs = Gc[cl * kN + n];  // what the later chunk hands back, entering through lane 15
            rb = fmaf(ra, gs * lastf, rb);
            scan16_down(rb, ra, gs);
            if (l == 0) Gc[cl * kN + n] = rb;  // handed to the earlier chunk
            // reverse, pass 2: g_t (the same FMA recurrence, now from what the right neighbour
            // hands this lane's last step) and every derivative of the step
            float pB[kK];
            float dAl = 0.f;
            {
                float Bv[kK];
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) *(float4 *)&Bv[4 * pc] = *(const float4 *)&Bc[n * kFP + pc * (kLPR * 4)];
                float gq = c[kK - 1] + gs;
#pragma unroll
                for (int j = kK - 1; j >= 0; --j) {
                    if (j < kK - 1) gq = fmaf(e[j + 1], gq, c[j]);
                    const float gw = gq * eh[j];
                    dAl = fmaf(dt[j], gw, dAl);
                    accdd[j] = fmaf(Araw, gw, accdd[j]);
                    if constexpr (ZOH) {
                        // input coefficient delta phi(y): d/d delta = e, d/dA = delta^2 phi'(y)
                        const float t = dt[j] * a2;
                        const float phi = zoh_phi(e[j], t);
                        const float dphi = zoh_dphi(e[j], t, phi);
                        const float gB = gq * Bv[j];
                        const float dlx = dt[j] * px[j];
                        accx[j] = fmaf(gB, phi, accx[j]);
                        pB[j] = gq * phi * dlx;
                        dAl = fmaf(gB, dlx * dt[j] * dphi, dAl);
                        accdd[j] = fmaf(px[j], e[j] * gB, accdd[j]);
                    } else {
                        accx[j] = fmaf(gq, Bv[j], accx[j]);
                        pB[j] = gq * px[j];
                    }
                }
            }
            {
                float r4[4];
                rows4_sum(pB, r4);
                *(float4 *)&redB[rslot] = make_float4(r4[0], r4[1], r4[2], r4[3]);
            }
            dAl = rowsum16(dAl);
            if (l == kLPR - 1) dAs[cl * kN + n] += dAl;
            clk.add(2);
            lds_barrier();
            clk.add(3);
            {
                // channel sums of this state's dB, dC for step tid of the chunk
                float sB = 0.f, sC = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    sB += red[w * kCH + rtid];
                    sC += red[4 * kCH + w * kCH + rtid];
                }
                if (s0 + tid < L) {
                    float *dst = p.wsBC + (((((int64_t)k * p.ntc + tc) * p.batch + b) * 2) * kN + n) * L + s0 + tid;
                    dst[0] = sB;
                    dst[(int64_t)kN * L] = sC;
                }
            }
            clk.add(2);
            lds_barrier();
            clk.add(4);
        }
        __builtin_amdgcn_s_setprio(2);

        // ---- per (step, channel) derivatives: dx, ddelta, and dz (or, with several directions,
        // this direction's output); they leave through three fp32 tiles: B, C (free after the
        // state loop) and the x/delta space (free once every wave has read it below)
        float dbl = 0.f;
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
            lds_barrier();  // every wave has read x and delta: their space takes the third tile
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
                float o0[4], o1[4], o2[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = 4 * pc + i;
                    float ddt = ZOH ? accdd[j] : fmaf(xf[j], accx[j], accdd[j]);
                    if (p.softplus) ddt *= sigmoidf_(df[j] + bias);
                    ddt = j < lim ? ddt : 0.f;
                    o0[i] = dt[j] * accx[j] + Dd * dyp[j];  // dx
                    o1[i] = ddt;                            // d(delta)
                    if constexpr (multi) {
                        o2[i] = yv[j];  // this direction's output; dz waits for the sum over directions
                    } else if (z) {
                        const float sg = sigmoidf_(zf[j]);
                        o2[i] = yf[j] * yv[j] * sg * (1.f + zf[j] * (1.f - sg));
                    } else {
                        o2[i] = 0.f;
                    }
                    dbl += ddt;
                }
                const int o = cl * kFP + pc * (kLPR * 4) + 4 * l;
                *(float4 *)&Bs[o] = make_float4(o0[0], o0[1], o0[2], o0[3]);
                *(float4 *)&Cs[o] = make_float4(o1[0], o1[1], o1[2], o1[3]);
                *(float4 *)&Os[o] = make_float4(o2[0], o2[1], o2[2], o2[3]);
            }
        }
        dDl = rowsum16(dDl);
        dbl = rowsum16(dbl);
        if (l == kLPR - 1) {
            dDs[2 * cl] += dDl;
            dDs[2 * cl + 1] += dbl;
        }
        lds_barrier();
        const bool want_z = z && p.dz;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int sl = so + 128 * r;
            const int64_t s = s0 + sl;
            if (nv <= 0 || s >= L) continue;
            const int64_t off = (rowb + visit<KIND>(p, k, s)) * dim + cg;
#pragma unroll
            for (int round = 0; round < 3; ++round) {
                if (round == 2 && !want_z) break;
                const float *tile = round == 0 ? Bs : (round == 1 ? Cs : Os);
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = tile[(8 * g + e) * kFP + fpos(sl)];
                if (round == 1) {
                    store8((T *)p.ddelta + k * tok + off, nv, vec, v);
                } else if constexpr (multi) {
                    // add the earlier directions' sum; keep it, or finish dx / dz
                    float *acc = (round == 0 ? p.wsX : p.wsY) + (split ? k * tok : 0);
                    if (k > 0 && !split) {
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
                        // opaque per chunk: otherwise the 16 per-lane addresses are hoisted out of
                        // every loop and spilled; this way the channel offsets are immediates
                        int xb = 8 * g * S::kXP + S::xpos(sl);
                        asm volatile("" : "+v"(xb));
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float dyv = Io<T>::f32(dyt[xb + e * S::kXP]);
                            const float zv = Io<T>::f32(zt[xb + e * S::kXP]);
                            const float sg = sigmoidf_(zv);
                            v[e] = dyv * v[e] * sg * (1.f + zv * (1.f - sg));
                        }
                        store8((T *)p.dz + off, nv, vec, v);
                    }
                } else {
                    store8((T *)(round == 0 ? p.dx : p.dz) + off, nv, vec, v);
                }
            }
        }
        clk.add(5);
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
#ifdef SELSCAN_PHASE_CLOCKS
    clk.finish(g_bwd_phase, blockIdx.x * 4 + wave, lane);
#endif
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
// with several directions the dx and pre-gate output sums (one row set, or one per direction
// for a split launch)
size_t bwd_ws_parts(int ndir, int64_t batch, int64_t L, int64_t dim, size_t part[5], bool split = false) {
    const int64_t ntc = (dim + kTC - 1) / kTC;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t K = (size_t)ndir;
    part[0] = up(K * (size_t)ntc * (size_t)batch * 2 * kN * (size_t)L * 4);
    part[1] = up(K * (size_t)batch * (size_t)dim * kN * 4);
    part[2] = up(K * (size_t)batch * (size_t)dim * 2 * 4);
    part[3] = part[4] = ndir > 1 ? up((split ? K : 1) * (size_t)batch * (size_t)L * (size_t)dim * 4) : 0;
    return part[0] + part[1] + part[2] + part[3] + part[4];
}

// Split launches: dx = ((dx_0 + dx_1) + ...) and, for the gate's derivative, the pre-gate output
// (o_0 + o_1) + ..., in direction order -- the sums the sequential walk forms -- then dz with
// the same expression as there.
struct BwdMergeParams {
    const float *wsX, *wsY;  // [ndir][batch * L][dim] partial rows
    const void *dy, *z;
    void *dx, *dz;
    int64_t rows, dim, tok;
    int ndir, vec, ncg;
};

template <typename T>
__global__ __launch_bounds__(256) void selscan_bwd_merge(BwdMergeParams m) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= m.rows * m.ncg) return;
    const int64_t row = gid / m.ncg, c0 = (gid % m.ncg) * 8;
    const int nv = (int)(m.dim - c0 < 8 ? m.dim - c0 : 8);
    const int64_t off = row * m.dim + c0;
    const bool vec = m.vec != 0;
    float s[8];
    load_f8(m.wsX + off, nv, vec, s);
    for (int k = 1; k < m.ndir; ++k) {
        float w[8];
        load_f8(m.wsX + k * m.tok + off, nv, vec, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = w[e] + s[e];
    }
    store8((T *)m.dx + off, nv, vec, s);
    if (m.dz) {
        load_f8(m.wsY + off, nv, vec, s);
        for (int k = 1; k < m.ndir; ++k) {
            float w[8];
            load_f8(m.wsY + k * m.tok + off, nv, vec, w);
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = w[e] + s[e];
        }
        const Raw8<T> dr = load_raw8((const T *)m.dy + off, nv, vec), zr = load_raw8((const T *)m.z + off, nv, vec);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float dyv = raw_f32(dr, e), zv = raw_f32(zr, e);
            const float sg = sigmoidf_(zv);
            s[e] = dyv * s[e] * sg * (1.f + zv * (1.f - sg));
        }
        store8((T *)m.dz + off, nv, vec, s);
    }
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
    bool split = false;  // decided from the workspace the caller gave (bwd_run)
};

// split when the grid would be short of workgroups and the workspace holds the per-direction rows
bool bwd_use_split(const BwdProblem &p, size_t ws_bytes) {
    size_t part[5];
    return p.ndir > 1 && split_wanted(p.kind, p.batch, p.dim) && p.ws &&
           ws_bytes >= bwd_ws_parts(p.ndir, p.batch, p.L, p.dim, part, true);
}

int bwd_validate(const BwdProblem &p, int64_t dstate, size_t ws_bytes) {
    if (p.batch < 0 || p.L < 0 || p.dim < 0 || p.H < 0 || p.W < 0 || dstate < 0) return SELSCAN_E_SHAPE;
    if (p.dtype != SELSCAN_F32 && p.dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (p.flags & ~(SELSCAN_FLAG_DELTA_SOFTPLUS | SELSCAN_FLAG_ZOH)) return SELSCAN_E_UNSUPPORTED;
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
    const size_t need = bwd_ws_parts(p.ndir, p.batch, p.L, p.dim, part, p.split);
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

template <typename T, int KIND, bool ZOH>
int bwd_launch_kind(const BwdProblem &q, void *stream) {
    BwdParams a;
    a.x = q.x, a.delta = q.delta, a.B = q.B, a.C = q.C, a.z = q.z, a.dy = q.dy;
    a.A = q.A, a.D = q.D, a.bias = q.bias, a.ckpt = q.ckpt;
    a.dx = q.dx, a.ddelta = q.ddelta, a.dz = q.z ? q.dz : nullptr, a.dh0 = q.dh0;
    size_t part[5];
    bwd_ws_parts(q.ndir, q.batch, q.L, q.dim, part, q.split);
    char *w = (char *)q.ws;
    a.wsBC = (float *)w;
    a.wsA = (float *)(w + part[0]);
    a.wsD = (float *)(w + part[0] + part[1]);
    a.wsX = q.ndir > 1 ? (float *)(w + part[0] + part[1] + part[2]) : nullptr;
    a.wsY = q.ndir > 1 ? (float *)(w + part[0] + part[1] + part[2] + part[3]) : nullptr;
    a.dim = q.dim;
    set_order(a, q.kind, q.L, q.H, q.W, q.win);
    a.batch = (int)q.batch, a.ndir = q.ndir;
    a.split = q.split ? 1 : 0;
    a.softplus = (q.flags & SELSCAN_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
    a.ntc = (int)((q.dim + kTC - 1) / kTC);
    const void *rows[] = {q.x, q.delta, q.dy, q.z, q.dx, q.ddelta, q.dz, a.wsX, a.wsY};
    bool vec = q.dim % 8 == 0;
    for (const void *r : rows)
        if (r && !aligned(r, 16)) vec = false;
    a.vec = vec;
    a.vecbc = aligned(q.B, 16) && aligned(q.C, 16);
    const int64_t blocks = q.batch * (int64_t)a.ntc * (a.split ? q.ndir : 1);
    if (blocks > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel((const void *)&selscan_bwd_chunked<T, KIND, ZOH>, dim3((unsigned)blocks), dim3(256),
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
    if (e == hipSuccess && a.split && q.L > 0) {
        BwdMergeParams m;
        m.wsX = a.wsX, m.wsY = a.wsY, m.dy = q.dy, m.z = q.z, m.dx = q.dx, m.dz = a.dz;
        m.rows = q.batch * q.L, m.dim = q.dim, m.tok = m.rows * q.dim;
        m.ndir = q.ndir, m.vec = a.vec, m.ncg = (int)((q.dim + 7) / 8);
        const int64_t mb = (m.rows * m.ncg + 255) / 256;
        if (mb > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
        void *margs[] = {&m};
        e = hipLaunchKernel((const void *)&selscan_bwd_merge<T>, dim3((unsigned)mb), dim3(256), margs, 0,
                            (hipStream_t)stream);
    }
    if (e != hipSuccess) {
        record_hip_error(e);
        return SELSCAN_E_HIP;
    }
    return SELSCAN_OK;
}

template <typename T, bool ZOH>
int bwd_launch_form(const BwdProblem &q, void *stream) {
    if (q.kind == SELSCAN_OP_FWD) return bwd_launch_kind<T, SELSCAN_OP_FWD, ZOH>(q, stream);
    if (q.kind == SELSCAN_OP_BIDIR) return bwd_launch_kind<T, SELSCAN_OP_BIDIR, ZOH>(q, stream);
    if (q.kind == SELSCAN_OP_SS2D) return bwd_launch_kind<T, SELSCAN_OP_SS2D, ZOH>(q, stream);
    return bwd_launch_kind<T, SELSCAN_OP_LOCAL_SS2D, ZOH>(q, stream);
}

template <typename T>
int bwd_launch(const BwdProblem &q, void *stream) {
    if (q.flags & SELSCAN_FLAG_ZOH) return bwd_launch_form<T, true>(q, stream);
    return bwd_launch_form<T, false>(q, stream);
}

int bwd_run(BwdProblem &p, int64_t dstate, size_t ws_bytes, void *stream) {
    p.split = bwd_use_split(p, ws_bytes);
    const int rc = bwd_validate(p, dstate, ws_bytes);
    if (rc != SELSCAN_OK) return rc;
    if (p.batch == 0 || p.dim == 0) return SELSCAN_OK;
    if (p.batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    if (p.dtype == SELSCAN_BF16) return bwd_launch<uint16_t>(p, stream);
    return bwd_launch<float>(p, stream);
}

}  // namespace

extern "C" {

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

#ifdef SELSCAN_PHASE_CLOCKS
// Diagnostic library only: copy the phase clocks of the last backward launch (8 u64 per wave,
// wave = 4 x workgroup + wave in workgroup: phases 0-5, whole kernel, 1 if written) to `host`,
// which holds `count` u64.  Returns 0, 1 if count is larger than the record, 2 on a HIP error.
int selscan_bwd_phase_read(unsigned long long *host, size_t count) {
    if (!host || count > (size_t)kPhaseWaves * 8) return 1;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_bwd_phase), count * sizeof(unsigned long long), 0,
                               hipMemcpyDeviceToHost) == hipSuccess ? 0 : 2;
}
// Clear the record (host-synchronous).
int selscan_bwd_phase_clear(void) {
    static const unsigned long long zeros[1024] = {};
    for (int i = 0; i < kPhaseWaves * 8; i += 1024)
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_bwd_phase), zeros, sizeof(zeros), i * sizeof(unsigned long long),
                              hipMemcpyHostToDevice) != hipSuccess)
            return 2;
    return 0;
}
#endif

size_t selscan_scan_bwd_workspace_bytes(int op, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                        int io_dtype) {
    (void)io_dtype;
    const int ndir = ndir_of(op);
    if (ndir == 0 || batch <= 0 || seqlen < 0 || dim <= 0 || dstate != kN) return 0;
    size_t part[5];
    return bwd_ws_parts(ndir, batch, seqlen, dim, part, ndir > 1 && split_wanted(op, batch, dim));
}

}  // extern "C"
