// libselscan - forward of the selective state-space scan for MI355X (gfx950) behind the C
// ABI declared in include/selscan.h (the backward is in selscan_bwd.hip).
//
// Method: "Mamba Series from Selective State Spaces to Visual State Space Models",
// section 选择性 SSM 的数学形式 (Abar = exp(delta A), selection of delta, B, C), insight 1
// (scan evaluated on chip with a parallel prefix scan, Abar/Bbar never written to HBM) and
// section 关键代码 (scan call with Ds, delta_bias, delta_softplus; the SS2D scan orders
// and merge; the SiLU gate); "从LSTM到Mamba" §2.1 (D skip) and §3.1 (bidirectional scan).
//
// Work decomposition (one kernel for every forward entry point):
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
#include "selscan_common.h"

#include <atomic>
#include <mutex>

namespace selscan_rt {
thread_local char g_last_hip_error[160] = "no error";
}  // namespace selscan_rt

// Device scratch of selscan_scan_fwd_noalloc (the partial-sum rows a multi-direction forward
// otherwise keeps in the caller's workspace).  Every GPU the library runs on holds one copy of
// this array until the process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// ------------------------------------------------------------------------------------
// host-side validation (pure host code: runs before any HIP call)
// ------------------------------------------------------------------------------------

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
    unsigned long long *stamps = nullptr;  // per workgroup: shader clock and real time at start and end
};

// the workspace a call would use: split when wanted and the caller's workspace holds it
size_t workspace_bytes_for(int op, int64_t batch, int64_t L, int64_t dim) {
    if (op == SELSCAN_OP_FWD) return 0;
    const size_t tok = (size_t)batch * (size_t)L * (size_t)dim * sizeof(float);
    return split_wanted(op, batch, dim) ? (size_t)ndir_of(op) * tok : tok;
}

size_t workspace_min_bytes(int op, int64_t batch, int64_t L, int64_t dim) {
    if (op == SELSCAN_OP_FWD) return 0;
    return (size_t)batch * (size_t)L * (size_t)dim * sizeof(float);
}

bool use_split(const Problem &p, size_t ws_bytes) {
    return p.ndir > 1 && split_wanted(p.kind, p.batch, p.dim) && p.ws &&
           ws_bytes >= workspace_bytes_for(p.kind, p.batch, p.L, p.dim);
}

int validate(const Problem &p, int64_t dstate, size_t ws_bytes) {
    if (p.batch < 0 || p.L < 0 || p.dim < 0 || p.H < 0 || p.W < 0 || dstate < 0) return SELSCAN_E_SHAPE;
    if (p.dtype != SELSCAN_F32 && p.dtype != SELSCAN_BF16) return SELSCAN_E_UNSUPPORTED;
    if (p.flags & ~(SELSCAN_FLAG_DELTA_SOFTPLUS | SELSCAN_FLAG_ZOH)) return SELSCAN_E_UNSUPPORTED;
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
    const size_t need = workspace_min_bytes(p.kind, p.batch, p.L, p.dim);
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
    // the workspace bytes the launch writes: one row set, or one per direction (split launches)
    size_t used = 0;
    if (need) {
        if (!p.ws || ws_bytes < need) return SELSCAN_E_WORKSPACE;
        used = use_split(p, ws_bytes) ? workspace_bytes_for(p.kind, p.batch, p.L, p.dim) : need;
        if (overlap(y, {p.ws, used})) return SELSCAN_E_ALIAS;
        for (int i = 0; i < 8; ++i)
            if (overlap({p.ws, used}, in[i])) return SELSCAN_E_ALIAS;
    }
    const Span wsu{used ? p.ws : nullptr, used};
    // state in/out: h_last may be h0 itself (in-place update) but must not overlap anything else
    const size_t st = (size_t)p.batch * (size_t)p.dim * kN * 4;
    if ((p.h0 && !aligned(p.h0, 4)) || (p.hlast && !aligned(p.hlast, 4))) return SELSCAN_E_ALIGN;
    const Span h0s{p.h0, st}, hls{p.hlast, st};
    if (overlap(y, h0s) || overlap(y, hls)) return SELSCAN_E_ALIAS;
    for (const Span &q : in)
        if (overlap(hls, q)) return SELSCAN_E_ALIAS;
    if (overlap(hls, wsu)) return SELSCAN_E_ALIAS;
    if (p.h0 != (const float *)p.hlast && overlap(hls, h0s)) return SELSCAN_E_ALIAS;
    if (p.ckpt) {
        const Span cks{p.ckpt, K * ckpt_bytes_for(p.batch, p.L, p.dim)};
        if (!aligned(p.ckpt, 4)) return SELSCAN_E_ALIGN;
        if (overlap(cks, y) || overlap(cks, h0s) || overlap(cks, hls) || overlap(cks, wsu)) return SELSCAN_E_ALIAS;
        for (const Span &q : in)
            if (overlap(cks, q)) return SELSCAN_E_ALIAS;
    }
    return SELSCAN_OK;
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
    int split;        // one direction per workgroup, partial sums per direction in ws
    int vec;          // rows of 8 channels may be moved as 16-byte vectors
    int vecbc;        // a 16-value B/C row may be moved as 16-byte vectors
    int ntc;          // channel tiles per batch row
    unsigned long long *stamps;  // NULL, or 4 counters per workgroup (selscan_scan_fwd_clocked)
};

// Shared-memory layout of a workgroup (16 channels), per chunk of kCH steps.  In every tile
// row the 16 steps of a lane are stored as 16-byte pieces: piece q of lane l sits at
// q * (16 lanes * piece) + l * piece, so that one 16-byte read by each of the 16 lanes of a
// row covers 256 contiguous bytes (no bank conflicts).  The scan reads A, D and bias of the
// current direction from one slot; those of a workgroup's later directions (up to KD - 1) wait
// in slots of their own.
template <typename T, int KD, int OCC = 2>
struct Lds {
    static constexpr int kCT = kTC;                                  // channels per tile
    static constexpr int kV = 16 / (int)sizeof(T);                    // io elements per piece
    static constexpr int kXP = kCH + kV;                              // io tile pitch (elements)
    static constexpr int kIoBytes = kCT * kXP * (int)sizeof(T);       // x or delta tile
    static constexpr int kYBytes = kCT * kFP * 4;                     // y tile fp32
    // bf16 io: the y tile has space of its own, so a wave writes its outputs without waiting
    // for the other waves to finish reading x and delta.  fp32 io, and the three-workgroup form:
    // y reuses the x/delta space (space of its own would leave room for one workgroup fewer per
    // compute unit).
    static constexpr bool kYOwn = sizeof(T) == 2 && OCC == 2;
    static constexpr int kXD = 2 * kIoBytes;
    static constexpr int kY = kYOwn ? kXD : 0;
    static constexpr int kB = kYOwn ? kXD + kYBytes : (kXD > kYBytes ? kXD : kYBytes);  // B [state][step]
    static constexpr int kC = kB + kN * kFP * 4;                      // C tile
    static constexpr int kA = kC + kN * kFP * 4;                      // A*log2e [ch][state]
    static constexpr int kCarry = kA + kCT * kN * 4;                  // chunk carry [ch][state]
    static constexpr int kDb = kCarry + kCT * kN * 4;                 // D, bias [ch][2]
    // later directions' A, D, bias (the three-workgroup form of the four-direction orders reads
    // them from memory at the direction switch instead: with them, three such workgroups would not
    // fit a CU)
    static constexpr bool kNoSlots = OCC == 3 && KD > 2;
    static constexpr int kSlots = kNoSlots ? 0 : KD - 1;
    static constexpr int kAx = kDb + kCT * 8;
    static constexpr int kDbx = kAx + kSlots * kCT * kN * 4;
    static constexpr int kBytes = kDbx + kSlots * kCT * 8;
    // position of chunk step s in an io tile row
    __device__ static int xpos(int s) { return ((s & 15) / kV) * (kLPR * kV) + (s >> 4) * kV + (s % kV); }
};
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

// The same scan for one state at a time (the three-workgroup form, whose waves have fewer
// registers): s_nop 1 before each DPP read of a value written by the instruction before it.
__device__ __forceinline__ void scan16(float &b, float &a, float &h) {
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
// Zero-order-hold input factor: zoh_phi (selscan_common.h).

#ifdef SELSCAN_PHASE_CLOCKS
// per-wave phase clocks of the forward (diagnostic library only): 0 staging (the barrier before,
// the wait for the chunk's loads, their commit to LDS, the barrier after), 1 the issue of the
// gate's and the next chunk's loads, 2 the prologue's arithmetic, 3 state loop, 4 the y tile's
// LDS writes and the barrier after them, 5 the output stores
__device__ unsigned long long g_fwd_phase[kPhaseWaves * 8];
#endif

// KK: scan steps per lane, 16 (chunks of 256 steps) or, for sequences of at most 16 KK steps,
// fewer (the sequence is one chunk): the LDS tiles keep 16 slots per lane, and slot 16 l + j
// holds chunk step KK l + j for j < KK (the slots past KK are left out everywhere).
// OCC: workgroups per compute unit the kernel is built for, 2 (the registers of two states at a
// time) or 3 (one state at a time, the y tile in the x/delta space, and for the four-direction
// orders no LDS slots for later directions' parameters; bf16 io, Euler Bbar and 16 steps per lane
// only).
template <typename T, int KIND, bool ZOH, int KK, int OCC = 2>
__global__ __launch_bounds__(256, OCC) void selscan_chunked(Params p) {
    constexpr int KD = KIND == SELSCAN_OP_FWD ? 1 : KIND == SELSCAN_OP_BIDIR ? 2 : 4;  // directions
    static_assert(OCC == 2 || (OCC == 3 && sizeof(T) == 2 && !ZOH && KK == kK),
                  "the three-workgroup form");
    using S = Lds<T, KD, OCC>;
    constexpr int CT = kTC;
    constexpr int NW = kN * (int)sizeof(T) / 4;  // dwords of one 16-value B or C row
    static_assert(CT * kN == 256, "one (channel, state) carry entry per thread");
    static_assert(KK >= 1 && KK <= kK, "steps per lane");
    constexpr int CHK = kLPR * KK;  // scan steps per chunk
    // chunk step of LDS slot s (valid when (s & 15) < KK) and slot of chunk step c
    auto cstep = [](int s) { return KK * (s >> 4) + (s & 15); };
    auto slot_of = [](int c) { return 16 * (c / KK) + c % KK; };
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::kBytes];
    // clock stamps (selscan_scan_fwd_clocked): shader-clock and 100 MHz real-time counters at the
    // workgroup's start (stored at once: nothing stays live across the kernel) and end
    if (p.stamps && threadIdx.x == 0) {
        unsigned long long *s = p.stamps + 4 * (int64_t)blockIdx.x;
        s[0] = __builtin_amdgcn_s_memtime();
        s[2] = __builtin_amdgcn_s_memrealtime();
    }
    T *xt = (T *)smem;
    T *dtl = (T *)(smem + S::kIoBytes);
    float *yt = (float *)(smem + S::kY);
    float *Bs = (float *)(smem + S::kB);
    float *Cs = (float *)(smem + S::kC);
    float *As = (float *)(smem + S::kA);
    float *Cy = (float *)(smem + S::kCarry);
    float *Db = (float *)(smem + S::kDb);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l = lane & 15;
    PhaseClock clk;
    const int cl = wave * 4 + (lane >> 4);     // this lane's channel within the tile
    // consecutive channel tiles on one XCD: workgroups are dealt round-robin over 8 XCDs
    const int G = gridDim.x, bi = blockIdx.x, q8 = G >> 3;
    const int tile_all = bi < (q8 << 3) ? (bi & 7) * q8 + (bi >> 3) : bi;
    // split launches: the grid is directions x tiles, each workgroup one direction of one tile
    constexpr bool multi = KIND != SELSCAN_OP_FWD;
    const int ntiles = p.batch * p.ntc;
    const bool split = multi && p.split;
    const int tile = split ? tile_all % ntiles : tile_all;
    const int b = tile / p.ntc;
    const int64_t c0 = (int64_t)(tile % p.ntc) * CT;
    const int64_t L = p.L, dim = p.dim;
    const int64_t tok = (int64_t)p.batch * L * dim, bcn = (int64_t)p.batch * L * kN;
    const int ncols = (int)(dim - c0 < CT ? dim - c0 : CT);
    const bool cvalid = cl < ncols;
    const int nchunks = (int)((L + CHK - 1) / CHK);
    const bool tile_fast = ncols == CT && p.vec && p.vecbc;  // full tile, vector rows
    const bool vec = p.vec != 0;
    const T *x = (const T *)p.x;
    const T *z = (const T *)p.z;
    T *y = (T *)p.y;
    const int64_t rowb = (int64_t)b * L;
    // a bidirectional sequence that fits one chunk, bf16 io: direction 0's y tile stays in its
    // LDS space and direction 1 adds it at its own output stage, so no partial-sum rows pass
    // through the fp32 workspace (the sum is the same: o_1 + o_0)
    bool lds_sum = false;
    if constexpr (KIND == SELSCAN_OP_BIDIR && S::kYOwn) lds_sum = !split && nchunks == 1;

    const int g = lane >> 5, nv = ncols - 8 * g;  // 8-channel group of the row items
    const int64_t cg = c0 + 8 * g;
    const int pp = 8 * (((lane >> 2) & 7) + 8 * (wave >> 1)) + 4 * (wave & 1) + (lane & 3);
    const int sb = 16 * (lane >> 2) + 4 * wave + (lane & 3);
    // zeros read by every lane but the first of a channel in place of the chunk carry
    __shared__ __attribute__((aligned(16))) float zero_pair[kN];
    if (tid < kN) zero_pair[tid] = 0.f;
    const float *carry_src = l == 0 ? Cy + cl * kN : zero_pair;
    const int so = 16 * ((lane >> 2) & 7) + 4 * wave + (lane & 3);

    int qq = 0;  // chunks done over all directions (priority parity)
    const int k_begin = split ? tile_all / ntiles : 0, k_end = split ? k_begin + 1 : multi ? p.ndir : 1;
    // A, D and bias of every direction of the workgroup, loaded once, in flight together with the
    // first chunk's loads; a later direction copies its own from LDS to the scan's slot at its
    // start instead of waiting on memory there.  The first chunk's fetch sits outside the
    // direction loop too: a single-direction kernel then has a loop of one known iteration,
    // and the compiler keeps fewer scalars alive (fewer spills into vector lanes).
    constexpr int KP = S::kNoSlots ? 1 : KD;  // directions whose parameters are loaded up front
    float av[KP], dv[KP], bv[KP];
    {
        const int ch = tid / kN, n = tid % kN;
        const int64_t cc = c0 + ch < dim ? c0 + ch : 0, cd = c0 + tid < dim ? c0 + tid : 0;
#pragma unroll
        for (int j = 0; j < KP; ++j) {
            const int k = k_begin + j;
            av[j] = dv[j] = bv[j] = 0.f;
            if (k < k_end && nchunks > 0) {
                av[j] = p.A[(k * dim + cc) * kN + n];
                if (tid < CT && p.D) dv[j] = p.D[k * dim + cd];
                if (tid < CT && p.bias) bv[j] = p.bias[k * dim + cd];
            }
        }
    }
    // global -> registers for one chunk, prefetched one chunk ahead (across directions too)
    Raw8<T> px0, px1, pd0, pd1;
    uint32_t pbc[2][NW];  // raw B and C values of one chunk step
    // chunk q of direction kk (reads the arguments the ordinary way: read afresh, the fetch
    // issued inside the state loop waited there on loads in flight into its address registers)
    auto fetch = [&](int kk, int q, auto fast_c) {
        const int64_t kt = multi ? kk : 0;
        const T *dl = (const T *)p.delta + kt * tok;
        const T *Bk = (const T *)p.B + kt * bcn;
        const T *Ck = (const T *)p.C + kt * bcn;
        const int64_t s0 = (int64_t)q * CHK;
        const int64_t sa = s0 + cstep(2 * pp), sbb = sa + 1, s = s0 + cstep(sb);
        // slots past KK in a lane hold no step
        const bool va = ((2 * pp) & 15) < KK, vb = ((2 * pp) & 15) + 1 < KK, vs = (sb & 15) < KK;
        if constexpr (decltype(fast_c)::value) {
            const int64_t oa = (rowb + visit<KIND>(p, kk, sa)) * dim + cg;
            const int64_t ob = (rowb + visit<KIND>(p, kk, sbb)) * dim + cg;
            const int64_t ro = (rowb + visit<KIND>(p, kk, s)) * kN;
            px0 = load_raw8(x + oa, 8, true);
            pd0 = load_raw8(dl + oa, 8, true);
            px1 = load_raw8(x + ob, 8, true);
            pd1 = load_raw8(dl + ob, 8, true);
#pragma unroll
            for (int h = 0; h < NW; h += 4) {
                const uint4 qb = *(const uint4 *)((const uint32_t *)(Bk + ro) + h);
                const uint4 qc = *(const uint4 *)((const uint32_t *)(Ck + ro) + h);
                pbc[0][h] = qb.x, pbc[0][h + 1] = qb.y, pbc[0][h + 2] = qb.z, pbc[0][h + 3] = qb.w;
                pbc[1][h] = qc.x, pbc[1][h + 1] = qc.y, pbc[1][h + 2] = qc.z, pbc[1][h + 3] = qc.w;
            }
        } else {
            px0 = px1 = pd0 = pd1 = Raw8<T>{};
            if (nv > 0 && va && sa < L) {
                const int64_t off = (rowb + visit<KIND>(p, kk, sa)) * dim + cg;
                px0 = load_raw8(x + off, nv, vec);
                pd0 = load_raw8(dl + off, nv, vec);
            }
            if (nv > 0 && vb && sbb < L) {
                const int64_t off = (rowb + visit<KIND>(p, kk, sbb)) * dim + cg;
                px1 = load_raw8(x + off, nv, vec);
                pd1 = load_raw8(dl + off, nv, vec);
            }
#pragma unroll
            for (int h = 0; h < NW; ++h) pbc[0][h] = pbc[1][h] = 0u;
            if (vs && s < L) {
                const int64_t ro = (rowb + visit<KIND>(p, kk, s)) * kN;
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
    fetch(k_begin, 0, BoolC<false>{});
    // read in the first direction's first chunk, after the barrier that follows its staging
#pragma unroll
    for (int j = 0; j < KP; ++j) {
        if (k_begin + j >= k_end) continue;
        float *a = j == 0 ? As : (float *)(smem + S::kAx) + (j - 1) * (CT * kN);
        float *d = j == 0 ? Db : (float *)(smem + S::kDbx) + (j - 1) * (2 * CT);
        a[tid] = av[j] * kLog2e;
        if (tid < CT) {
            d[2 * tid] = dv[j];
            d[2 * tid + 1] = bv[j];
        }
    }
    for (int k = k_begin; k < k_end; ++k) {
        // the previous direction is done with the parameter tiles and the carry, and its stores
        // of the partial sums (which other waves read back in this direction) are complete: a
        // full barrier
        __syncthreads();
        if (k > k_begin) {
            if constexpr (S::kNoSlots) {
                const int ch = tid / kN, n = tid % kN;
                const int64_t cc = c0 + ch < dim ? c0 + ch : 0, cd = c0 + tid < dim ? c0 + tid : 0;
                As[tid] = p.A[(k * dim + cc) * kN + n] * kLog2e;
                if (tid < CT) {
                    Db[2 * tid] = p.D ? p.D[k * dim + cd] : 0.f;
                    Db[2 * tid + 1] = p.bias ? p.bias[k * dim + cd] : 0.f;
                }
            } else {
                const int j = k - k_begin - 1;
                As[tid] = ((const float *)(smem + S::kAx))[j * (CT * kN) + tid];
                if (tid < 2 * CT) Db[tid] = ((const float *)(smem + S::kDbx))[j * (2 * CT) + tid];
            }
        }
        for (int i = tid; i < CT * kN; i += 256) {
            const int ch = i / kN, n = i % kN;
            // the carry into the first chunk: the caller's initial state, else zero
            Cy[i] = p.h0 && c0 + ch < dim ? p.h0[((int64_t)b * dim + c0 + ch) * kN + n] : 0.f;
        }

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
            // the arguments, read afresh in every chunk (fresh_args); not for the windowed orders,
            // whose index map reads four divisions, where that spills more than it saves
            auto &args = [&]() -> auto & {
                if constexpr (KIND == SELSCAN_OP_LOCAL_SS2D) return p;
                else return fresh_args<Params>();
            }();
            const int64_t s0 = (int64_t)q * CHK;
            __builtin_amdgcn_s_setprio(2);
            // the previous chunk is done with every tile (a one-chunk sequence's only chunk of a
            // direction follows the direction's opening barrier, which covers this).  Where the y
            // tile has LDS space of its own, the previous chunk's y-tile barrier already follows
            // every wave's last read of the tiles written here (its state loop comes first), so
            // only the fp32 form, whose y tile sits in the x/delta space, waits here.
            if constexpr (KK == kK && !S::kYOwn) lds_barrier();
            commit();
            lds_barrier();
            clk.add(0);
            if (args.ckpt) {
                // the carry entering this chunk, kept for the backward pass
                const int ch = tid / kN, n = tid % kN;
                if (c0 + ch < dim)
                    args.ckpt[((((int64_t)k * args.batch + b) * nchunks + q) * dim + c0 + ch) * kN + n] = Cy[tid];
            }
            // gate input for this chunk's output items, then the next chunk's inputs, in flight while
            // this chunk computes.  A single-direction scan with 16 steps per lane issues them after
            // the state loop's first state pair: issued right after the chunk-start barrier, every
            // wave of the workgroup queued its loads at once and waited on the memory pipeline for
            // ~11 % of the kernel; one state pair later the waves have drifted apart.  The other
            // forms issue them here, as written out below: they measured no gain from the later
            // issue, and even calling the same code through the lambda here changes their register
            // allocation (more spills, Vim 2 % slower).
            const bool last = k == args.ndir - 1 && !split;
            float *wsk = split ? args.ws + k * tok : args.ws;  // this direction's partial rows (split) or the running sum
            Raw8<T> zr[2];  // read only where it was loaded
            int64_t ooff[2] = {0, 0};
            constexpr bool mid_issue = KIND == SELSCAN_OP_FWD && KK == kK && sizeof(T) == 2 && !ZOH;
            // the three-workgroup form issues them after the state loop: its registers do not
            // hold the loaded rows, or z, across the loop (issued in the loop, z alone spilled 21
            // more VGPRs; the rows as well, 39)
            constexpr bool late_issue = OCC == 3;
            auto issue_z = [&]() {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int64_t s = s0 + cstep(so + 128 * r);
                    if constexpr (fast) {
                        ooff[r] = (rowb + visit<KIND>(args, k, s)) * dim + cg;
                        if (last && z) zr[r] = load_raw8(z + ooff[r], 8, true);
                    } else {
                        zr[r] = Raw8<T>{};
                        if (nv > 0 && ((so + 128 * r) & 15) < KK && s < L) {
                            ooff[r] = (rowb + visit<KIND>(args, k, s)) * dim + cg;
                            if (last && z) zr[r] = load_raw8(z + ooff[r], nv, vec);
                        }
                    }
                }
            };
            auto issue_next = [&]() {
                if constexpr (fast || !multi) {
                    if (q + 1 < nchunks) fetch(k, q + 1, fast_c);
                } else {
                    // after a direction's last chunk, the next direction's first
                    const bool next_dir = q + 1 == nchunks;
                    if (!next_dir || k + 1 < k_end) fetch(next_dir ? k + 1 : k, next_dir ? 0 : q + 1, fast_c);
                }
            };
            auto issue_loads = [&]() {
                issue_z();
                issue_next();
            };
            if constexpr (!mid_issue && !late_issue) {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int64_t s = s0 + cstep(so + 128 * r);
                    if constexpr (fast) {
                        ooff[r] = (rowb + visit<KIND>(args, k, s)) * dim + cg;
                        if (last && z) zr[r] = load_raw8(z + ooff[r], 8, true);
                    } else {
                        zr[r] = Raw8<T>{};
                        if (nv > 0 && ((so + 128 * r) & 15) < KK && s < L) {
                            ooff[r] = (rowb + visit<KIND>(args, k, s)) * dim + cg;
                            if (last && z) zr[r] = load_raw8(z + ooff[r], nv, vec);
                        }
                    }
                }
                if constexpr (fast || !multi) {
                    if (q + 1 < nchunks) fetch(k, q + 1, fast_c);
                } else {
                    // after a direction's last chunk, the next direction's first
                    const bool next_dir = q + 1 == nchunks;
                    if (!next_dir || k + 1 < k_end) fetch(next_dir ? k + 1 : k, next_dir ? 0 : q + 1, fast_c);
                }
            }

            clk.add(1);
            // ---- this lane's KK steps of its channel
            const int64_t rem = L - (s0 + l * KK);
            const int lim = !cvalid ? 0 : (rem <= 0 ? 0 : (rem >= KK ? KK : (int)rem));
            float dt[KK], dx[KK], yv[KK];
            float sdt = 0.f;
            {
                const float Dd = Db[2 * cl];
                float xf[KK];
                constexpr int V = S::kV;
#pragma unroll
                for (int pc = 0; pc < (KK + V - 1) / V; ++pc) {
                    const uint4 xq = *(const uint4 *)&xt[cl * S::kXP + pc * (kLPR * V) + l * V];
                    const uint4 dq = *(const uint4 *)&dtl[cl * S::kXP + pc * (kLPR * V) + l * V];
                    const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w}, dw[4] = {dq.x, dq.y, dq.z, dq.w};
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        if (pc * V + i >= KK) continue;
                        if constexpr (sizeof(T) == 2) {
                            xf[pc * V + i] = __uint_as_float(i & 1 ? xw[i >> 1] & 0xFFFF0000u : xw[i >> 1] << 16);
                            dt[pc * V + i] = __uint_as_float(i & 1 ? dw[i >> 1] & 0xFFFF0000u : dw[i >> 1] << 16);
                        } else {
                            xf[pc * V + i] = __uint_as_float(xw[i]);
                            dt[pc * V + i] = __uint_as_float(dw[i]);
                        }
                    }
                }
                // bias, then softplus, in place (one set of registers for every form)
                if (args.bias) {
                    const float bias = Db[2 * cl + 1];
#pragma unroll
                    for (int j = 0; j < KK; ++j) dt[j] += bias;
                }
                if (args.softplus) {
#pragma unroll
                    for (int j = 0; j < KK; ++j) dt[j] = softplus(dt[j]);
                }
                if (!fast && !(s0 + CHK <= L && ncols == CT) && (args.bias || args.softplus)) {
                    // steps past the sequence end and channels past dim get delta = 0, the
                    // identity step (staged x there is 0 too).  Staging leaves zeros there, so
                    // only a bias or softplus (which move 0) needs the mask.
                    const float limf = (float)lim;
#pragma unroll
                    for (int j = 0; j < KK; ++j) dt[j] *= __builtin_amdgcn_fmed3f(limf - (float)j, 0.f, 1.f);
                }
#pragma unroll
                for (int j = 0; j < KK; ++j) {
                    dx[j] = dt[j] * xf[j];
                    yv[j] = Dd * xf[j];
                    sdt += dt[j];
                }
            }
            if (qq & 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            clk.add(2);
            const float *Bc = Bs + 4 * l;
            const float *Cc = Cs + 4 * l;
            if constexpr (OCC == 3) {
                // one state at a time
#pragma unroll 1
                for (int n = 0; n < kN; ++n) {
                    const float an = As[cl * kN + n];
                    float e[kK], u[kK], bb;
                    {
                        float Bv[kK];
#pragma unroll
                        for (int pc = 0; pc < kK / 4; ++pc)
                            *(float4 *)&Bv[4 * pc] = *(const float4 *)&Bc[n * kFP + pc * (kLPR * 4)];
#pragma unroll
                        for (int j = 0; j < kK; ++j) {
                            e[j] = __builtin_amdgcn_exp2f(dt[j] * an);
                            u[j] = dx[j] * Bv[j];
                            bb = j == 0 ? u[0] : fmaf(e[j], bb, u[j]);  // from a zero state
                        }
                    }
                    float a = __builtin_amdgcn_exp2f(an * sdt);
                    float h = carry_src[n];  // the channel's carry in its first lane, else zero
                    bb = fmaf(a, h, bb);
                    scan16(bb, a, h);
                    if (l == kLPR - 1) Cy[cl * kN + n] = bb;
                    float Cv[kK];
#pragma unroll
                    for (int pc = 0; pc < kK / 4; ++pc)
                        *(float4 *)&Cv[4 * pc] = *(const float4 *)&Cc[n * kFP + pc * (kLPR * 4)];
#pragma unroll
                    for (int j = 0; j < kK; ++j) {
                        h = fmaf(e[j], h, u[j]);
                        yv[j] = fmaf(Cv[j], h, yv[j]);
                    }
                }
                if constexpr (late_issue) issue_loads();
            } else {
#pragma unroll 1
            for (int n = 0; n < kN; n += 2) {
                if constexpr (mid_issue) {
                    if (n == 2) issue_loads();
                }
                const float2 a2 = *(const float2 *)&As[cl * kN + n];
                constexpr int NP = (KK + 3) / 4;  // 4-step pieces of a lane's slots that hold steps
                float e0[KK], u0[KK], e1[KK], u1[KK];
                float b0, b1;
                {
                    float B0[4 * NP], B1[4 * NP];
#pragma unroll
                    for (int pc = 0; pc < NP; ++pc) {
                        *(float4 *)&B0[4 * pc] = *(const float4 *)&Bc[n * kFP + pc * (kLPR * 4)];
                        *(float4 *)&B1[4 * pc] = *(const float4 *)&Bc[(n + 1) * kFP + pc * (kLPR * 4)];
                    }
#pragma unroll
                    for (int j = 0; j < KK; ++j) {
                        const float t0 = dt[j] * a2.x, t1 = dt[j] * a2.y;
                        e0[j] = __builtin_amdgcn_exp2f(t0);
                        e1[j] = __builtin_amdgcn_exp2f(t1);
                        if constexpr (ZOH) {
                            u0[j] = dx[j] * zoh_phi(e0[j], t0) * B0[j];
                            u1[j] = dx[j] * zoh_phi(e1[j], t1) * B1[j];
                        } else {
                            u0[j] = dx[j] * B0[j];
                            u1[j] = dx[j] * B1[j];
                        }
                        b0 = j == 0 ? u0[0] : fmaf(e0[j], b0, u0[j]);  // from a zero state
                        b1 = j == 0 ? u1[0] : fmaf(e1[j], b1, u1[j]);
                    }
                }
                float a0 = __builtin_amdgcn_exp2f(a2.x * sdt);
                float a1 = __builtin_amdgcn_exp2f(a2.y * sdt);
                // the previous chunk's end state of this channel enters through its first lane
                // (the other lanes read zeros)
                const float2 cy = *(const float2 *)&carry_src[n];
                float h0 = cy.x, h1 = cy.y;
                b0 = fmaf(a0, h0, b0);
                b1 = fmaf(a1, h1, b1);
                scan16x2(b0, b1, a0, a1, h0, h1);
                // the last lane of a channel holds the chunk's end state: the next chunk's carry
                if (l == kLPR - 1) *(float2 *)&Cy[cl * kN + n] = make_float2(b0, b1);
                float C0[4 * NP], C1[4 * NP];
#pragma unroll
                for (int pc = 0; pc < NP; ++pc) {
                    *(float4 *)&C0[4 * pc] = *(const float4 *)&Cc[n * kFP + pc * (kLPR * 4)];
                    *(float4 *)&C1[4 * pc] = *(const float4 *)&Cc[(n + 1) * kFP + pc * (kLPR * 4)];
                }
#pragma unroll
                for (int j = 0; j < KK; ++j) {
                    h0 = fmaf(e0[j], h0, u0[j]);
                    h1 = fmaf(e1[j], h1, u1[j]);
                    yv[j] = fmaf(C0[j], h0, yv[j]);
                    yv[j] = fmaf(C1[j], h1, yv[j]);
                }
            }
            }
            __builtin_amdgcn_s_setprio(2);
            clk.add(3);
            // direction 1 of an LDS-summed pair writes its tile into the x/delta space
            const bool y_in_xd = lds_sum && k == 1;
            if constexpr (!S::kYOwn) lds_barrier();  // x/delta tiles fully read before y reuses their space
            else if (y_in_xd) lds_barrier();
            float *yw = y_in_xd ? (float *)smem : yt;
#pragma unroll
            for (int pc = 0; pc < (KK + 3) / 4; ++pc) {
                // (slots past KK are written with zeros and never read)
                float q4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) q4[i] = 4 * pc + i < KK ? yv[4 * pc + i] : 0.f;
                *(float4 *)&yw[cl * kFP + pc * (kLPR * 4) + 4 * l] = make_float4(q4[0], q4[1], q4[2], q4[3]);
            }
            // the gate of this chunk's output items, ahead of the barrier, with 16 steps per lane: a
            // wave that reaches it early computes its gates while the others finish their state
            // loops (the one-chunk form measured slower with it, and gates after the barrier)
            constexpr bool early_gate = KK == kK;
            float gz[2][8];
            if (early_gate && last && z) {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) gz[r][e] = silu(raw_f32(zr[r], e));
                }
            }
            lds_barrier();
            clk.add(4);
            if (lds_sum && k == 0) return;  // direction 0's tile waits in LDS for direction 1
            // ---- leave: add earlier directions, gate, store y (or keep the partial sum)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int sl = so + 128 * r;
                float v[8], wv[8];
                if constexpr (fast) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = yt[(8 * g + e) * kFP + fpos(sl)];
                    if (multi && k > 0 && !split) {
                        load_f8(args.ws + ooff[r], 8, true, wv);
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] += wv[e];
                    }
                    if (last && z) {
                        // the gated and the ungated store are separate calls: no register copies
                        // where the two forms would join
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] *= early_gate ? gz[r][e] : silu(raw_f32(zr[r], e));
                        store8(y + ooff[r], 8, true, v);
                    } else if (last) {
                        store8(y + ooff[r], 8, true, v);
                    } else {
                        store8(wsk + ooff[r], 8, true, v);
                    }
                } else if (nv > 0 && (sl & 15) < KK && s0 + cstep(sl) < L) {
                    if (y_in_xd) {
                        // this direction's step c (slot sl) is token L-1-c, direction 0's step L-1-c
                        const int sl0 = slot_of((int)L - 1 - cstep(sl));
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            v[e] = yw[(8 * g + e) * kFP + fpos(sl)];
                            wv[e] = yt[(8 * g + e) * kFP + fpos(sl0)];
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = yt[(8 * g + e) * kFP + fpos(sl)];
                        if (multi && k > 0 && !split) load_f8(args.ws + ooff[r], nv, vec, wv);
                    }
                    if (multi && (y_in_xd || (k > 0 && !split))) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] += wv[e];
                    }
                    if (last) {
                        if (z) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] *= early_gate ? gz[r][e] : silu(raw_f32(zr[r], e));
                        }
                        store8(y + ooff[r], nv, vec, v);
                    } else {
                        store8(wsk + ooff[r], nv, vec, v);
                    }
                }
            }
            clk.add(5);
        };
        clk.mark();
        const int nfast = tile_fast && KK == kK ? (int)(L / CHK) - 1 : 0;
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
    if (p.stamps && threadIdx.x == 0) {
        unsigned long long *s = p.stamps + 4 * (int64_t)blockIdx.x;
        s[1] = __builtin_amdgcn_s_memtime();
        s[3] = __builtin_amdgcn_s_memrealtime();
    }
#ifdef SELSCAN_PHASE_CLOCKS
    clk.finish(g_fwd_phase, blockIdx.x * 4 + wave, lane);
#endif
}

// Split launches: y = (((o_0 + o_1) + o_2) + o_3) * silu(z) from the per-direction partial rows
// -- the sums the sequential walk forms, in its order (fp32 addition is commutative).
struct MergeParams {
    const float *ws;  // [ndir][batch * L][dim] partial outputs
    const void *z;
    void *y;
    int64_t rows, dim, tok;  // rows = batch * L; tok = rows * dim
    int ndir, vec, ncg;
};

template <typename T>
__global__ __launch_bounds__(256) void selscan_merge(MergeParams m) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= m.rows * m.ncg) return;
    const int64_t row = gid / m.ncg, c0 = (gid % m.ncg) * 8;
    const int nv = (int)(m.dim - c0 < 8 ? m.dim - c0 : 8);
    const int64_t off = row * m.dim + c0;
    const bool vec = m.vec != 0;
    float s[8];
    load_f8(m.ws + off, nv, vec, s);
    for (int k = 1; k < m.ndir; ++k) {
        float w[8];
        load_f8(m.ws + k * m.tok + off, nv, vec, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = w[e] + s[e];
    }
    if (m.z) {
        const Raw8<T> zr = load_raw8((const T *)m.z + off, nv, vec);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] *= silu(raw_f32(zr, e));
    }
    store8((T *)m.y + off, nv, vec, s);
}

// The three-workgroup form for a grid of `blocks` workgroups on a device of `cus` compute units.
// Rounds of workgroups: r2 = ceil(blocks / 2 cus) for the two-workgroup form, r3 = ceil(blocks /
// 3 cus) for this one, whose round takes longer (one state at a time, loads issued after the state
// loop, a third barrier); it is launched where 1.25 r3 < r2.  A sweep of the scan order (bf16, 2,048
// steps, 1.5 to 9 workgroups per unit, 200 warm-up launches) put the break-even ratio between 1.0
// and 1.33 for every grid size measured: e.g. 2.25-3 per unit 0.125 -> 0.105-0.108 ms, 3.4-3.75 per
// unit 0.145-0.149 (two-workgroup form) against 0.155-0.159, 9 per unit 0.358 -> 0.331 ms; one
// round of either (the Mamba-1.4B layer's 512 workgroups) keeps the two-workgroup form.  The
// multi-direction orders take the same rule (direction-split grids of 1,536 workgroups: VideoMamba
// clip 0.264 -> 0.252 ms, SS2D map 0.478 -> 0.453, windowed map 0.482 -> 0.458 ms with the merge).
bool occ3_wanted(int64_t blocks, int cus) {
#ifdef SELSCAN_OCC3_ALWAYS
    (void)blocks, (void)cus;
    return true;
#else
    if (cus <= 0) return false;
    const int64_t r2 = (blocks + 2 * (int64_t)cus - 1) / (2 * (int64_t)cus);
    const int64_t r3 = (blocks + 3 * (int64_t)cus - 1) / (3 * (int64_t)cus);
    return 5 * r3 < 4 * r2;
#endif
}

// compute units of the device that `stream` launches on (0 if unknown), cached per device
int stream_cus(void *stream) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return 0;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return 0;
    }
    constexpr int kDevs = 64;
    static std::atomic<int> cache[kDevs];  // zero: not yet asked
    if (dev < 0 || dev >= kDevs) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <typename T, int KIND>
int launch_tiles(const Params &a, int64_t batch, bool zoh, void *stream) {
    Params c = a;
    c.ntc = (int)((a.dim + kTC - 1) / kTC);
    const int64_t blocks = batch * (int64_t)c.ntc * (c.split ? c.ndir : 1);
    if (blocks > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    void *args[] = {&c};
    // a sequence of at most 208 steps is one chunk of 13 steps per lane (Euler Bbar); else 16
    const bool short13 = !zoh && c.L <= kLPR * 13;
    const void *kern = zoh ? (const void *)&selscan_chunked<T, KIND, true, kK>
                           : short13 ? (const void *)&selscan_chunked<T, KIND, false, 13>
                                     : (const void *)&selscan_chunked<T, KIND, false, kK>;
    if constexpr (sizeof(T) == 2) {
        if (!zoh && !short13 && occ3_wanted(blocks, stream_cus(stream)))
            kern = (const void *)&selscan_chunked<T, KIND, false, kK, 3>;
    }
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)blocks), dim3(256), args, 0, (hipStream_t)stream);
    if (e == hipSuccess && c.split && c.L > 0) {
        MergeParams m;
        m.ws = c.ws, m.z = c.z, m.y = c.y;
        m.rows = (int64_t)batch * c.L, m.dim = c.dim, m.tok = m.rows * c.dim;
        m.ndir = c.ndir, m.vec = c.vec, m.ncg = (int)((c.dim + 7) / 8);
        const int64_t mb = (m.rows * m.ncg + 255) / 256;
        if (mb > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
        void *margs[] = {&m};
        e = hipLaunchKernel((const void *)&selscan_merge<T>, dim3((unsigned)mb), dim3(256), margs, 0, (hipStream_t)stream);
    }
    if (e != hipSuccess) {
        record_hip_error(e);
        return SELSCAN_E_HIP;
    }
    return SELSCAN_OK;
}

template <typename T>
int launch_kind(const Params &a, int kind, int64_t batch, bool zoh, void *stream) {
    if (kind == SELSCAN_OP_FWD) return launch_tiles<T, SELSCAN_OP_FWD>(a, batch, zoh, stream);
    if (kind == SELSCAN_OP_BIDIR) return launch_tiles<T, SELSCAN_OP_BIDIR>(a, batch, zoh, stream);
    if (kind == SELSCAN_OP_SS2D) return launch_tiles<T, SELSCAN_OP_SS2D>(a, batch, zoh, stream);
    return launch_tiles<T, SELSCAN_OP_LOCAL_SS2D>(a, batch, zoh, stream);
}

int launch(const Problem &p, size_t ws_bytes, void *stream) {
    Params a;
    a.x = p.x, a.delta = p.delta, a.B = p.B, a.C = p.C, a.z = p.z;
    a.A = p.A, a.D = p.D, a.bias = p.bias, a.y = p.y;
    a.ws = p.ndir > 1 ? (float *)p.ws : nullptr;
    a.h0 = p.h0, a.hlast = p.hlast, a.ckpt = p.ckpt;
    a.dim = p.dim;
    set_order(a, p.kind, p.L, p.H, p.W, p.win);
    a.batch = (int)p.batch, a.ndir = p.ndir;
    a.split = use_split(p, ws_bytes) ? 1 : 0;
    a.softplus = (p.flags & SELSCAN_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
    // rows of 8 channels move as 16-byte vectors when every row start is 16-byte aligned
    const void *rows[] = {p.x, p.delta, p.z, p.y};
    bool vec = p.dim % 8 == 0 && (!a.ws || aligned(a.ws, 16));
    for (const void *q : rows)
        if (q && !aligned(q, 16)) vec = false;
    a.vec = vec;
    a.vecbc = aligned(p.B, 16) && aligned(p.C, 16);
    a.ntc = 0;
    a.stamps = p.stamps;
    const bool zoh = (p.flags & SELSCAN_FLAG_ZOH) != 0;
    if (p.dtype == SELSCAN_BF16) return launch_kind<uint16_t>(a, p.kind, p.batch, zoh, stream);
    return launch_kind<float>(a, p.kind, p.batch, zoh, stream);
}

int run(Problem &p, int64_t dstate, size_t ws_bytes, void *stream) {
    int rc = validate(p, dstate, ws_bytes);
    if (rc != SELSCAN_OK) return rc;
    if (p.batch == 0 || p.dim == 0 || (p.L == 0 && !p.hlast)) return SELSCAN_OK;
    if (p.batch > 0x7FFFFFFF) return SELSCAN_E_UNSUPPORTED;
    return launch(p, ws_bytes, stream);
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

int selscan_scan_fwd_clocked(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                             const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                             float *chunk_states, int64_t batch, int64_t seqlen, int64_t H, int64_t W,
                             int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *workspace,
                             size_t workspace_bytes, unsigned long long *stamps, void *stream) {
    if (!stamps) return SELSCAN_E_NULL;
    if (!aligned(stamps, 8)) return SELSCAN_E_ALIGN;
    int64_t L;
    int ndir;
    const int rc = resolve_op(op, seqlen, H, W, &L, &ndir);
    if (rc != SELSCAN_OK) return rc;
    const bool two_d = op == SELSCAN_OP_SS2D || op == SELSCAN_OP_LOCAL_SS2D;
    Problem p{x,     delta, B, C, z, A, D, delta_bias, y, workspace, batch, L, dim, two_d ? H : 0, two_d ? W : 0,
              ndir,  op,    io_dtype, flags};
    p.ckpt = chunk_states;
    p.win = op == SELSCAN_OP_LOCAL_SS2D ? window : 0;
    p.stamps = stamps;
    return run(p, dstate, workspace_bytes, stream);
}

#ifdef SELSCAN_PHASE_CLOCKS
// Diagnostic library only: copy the phase clocks of the last forward launch (8 u64 per wave,
// wave = 4 x workgroup + wave in workgroup: phases 0-5, whole kernel, 1 if written) to
// `host`, which holds `count` u64.  Returns 0, 1 if count is larger than the record, 2 on a HIP
// error.
int selscan_fwd_phase_read(unsigned long long *host, size_t count) {
    if (!host || count > (size_t)kPhaseWaves * 8) return 1;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_fwd_phase), count * sizeof(unsigned long long), 0,
                               hipMemcpyDeviceToHost) == hipSuccess ? 0 : 2;
}
// Clear the record (host-synchronous).
int selscan_fwd_phase_clear(void) {
    static const unsigned long long zeros[1024] = {};
    for (int i = 0; i < kPhaseWaves * 8; i += 1024)
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_fwd_phase), zeros, sizeof(zeros), i * sizeof(unsigned long long),
                              hipMemcpyHostToDevice) != hipSuccess)
            return 2;
    return 0;
}
#endif

size_t selscan_clock_stamps_bytes(int op, int64_t batch, int64_t dim) {
    const int ndir = ndir_of(op);
    if (ndir == 0 || batch <= 0 || dim <= 0) return 0;
    return (size_t)batch * (size_t)((dim + kTC - 1) / kTC) * (size_t)ndir * 4 * sizeof(unsigned long long);
}

size_t selscan_scan_chunk_states_bytes(int op, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
    const int ndir = ndir_of(op);
    if (ndir == 0 || batch <= 0 || seqlen <= 0 || dim <= 0 || dstate != kN) return 0;
    return (size_t)ndir * ckpt_bytes_for(batch, seqlen, dim);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// The device a launch on `stream` runs on: the stream's own device, or the current device for the
// null stream.
int stream_device(void *stream, int *dev) {
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, dev) : hipGetDevice(dev);
    if (e != hipSuccess) {
        record_hip_error(e);
        return SELSCAN_E_HIP;
    }
    return SELSCAN_OK;
}

// Device address of `scratch` on device `dev`, looked up on the first call for that device with
// that device current (the caller's current device is restored) and kept for later calls.
int scratch_on(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return SELSCAN_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void *p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess || !p) {
            record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return SELSCAN_E_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SELSCAN_OK;
}

}  // namespace

extern "C" {

int selscan_scan_fwd_noalloc(int op, const void *x, const void *delta, const float *A, const void *B, const void *C,
                             const float *D, const void *z, const float *delta_bias, unsigned flags, void *y,
                             float *chunk_states, int64_t batch, int64_t seqlen, int64_t H, int64_t W,
                             int64_t window, int64_t dim, int64_t dstate, int io_dtype, void *stream) {
    int64_t L;
    int ndir;
    int rc = resolve_op(op, seqlen, H, W, &L, &ndir);
    if (rc != SELSCAN_OK) return rc;
    // the workspace this call needs must fit the static array (one row set at least; the
    // per-direction rows of a split launch when they fit too)
    if (batch > 0 && dim > 0 && L > 0 && workspace_min_bytes(op, batch, L, dim) > kScratchBytes)
        return SELSCAN_E_WORKSPACE;
    void *ws = nullptr;
    if (ndir > 1 && batch > 0 && dim > 0 && L > 0) {
        int dev = 0;
        rc = stream_device(stream, &dev);
        if (rc != SELSCAN_OK) return rc;
        rc = scratch_on(dev, &ws);
        if (rc != SELSCAN_OK) return rc;
    }
    return selscan_scan_fwd(op, x, delta, A, B, C, D, z, delta_bias, flags, y, chunk_states, batch, seqlen, H, W,
                            window, dim, dstate, io_dtype, ws, ws ? kScratchBytes : 0, stream);
}

size_t selscan_scan_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

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

const char *selscan_last_hip_error(void) { return selscan_rt::g_last_hip_error; }

}  // extern "C"
