// Linear-layer GEMM family for MI355X (gfx950): HIP kernels + C ABI.
//
// Operations ("matmul ve matmul_residual — Tiled Matrix Multiply (Forward)",
// https://llm.istanbul/learn/tr/03_linear_forward, section "Ne Yapar?"):
//   Y = A @ W (+ R),  A = X  or  A = silu(GATE) * UP,  W fp32 or binary16,
// and the backward kernels the same section names: dX = dY @ W^T
// (matmul_t), dW = A^T @ dY (matmul_at, A recomputed as silu(GATE) * UP for
// _swiglu_a), each optionally accumulating into the output (_acc), plus
// matmul_t with the SwiGLU backward fused into its epilogue.
//
// Design (gfx950, wave64, fp32 matrix cores):
//  * One workgroup owns one BM x BN output tile over its K range (the page's
//    "Tile Hiyerarşisi").  On small output grids the K range of a tile is
//    split over KS workgroups whose fp32 partial tiles meet in a static
//    workspace and are added in the fixed order 0..KS-1, so every run gives
//    the same bits whatever order the workgroups finish in.
//  * The contraction runs on v_mfma_f32_16x16x4_f32.  Within a 16-wide slice
//    of K each lane feeds four consecutive k values (one float4) to four
//    MFMAs; the pairing of k with lanes is the same for A and B, so the sum
//    covers every k exactly once.
//  * A and W tiles are staged through LDS in their global orientation: A
//    k-contiguous with its float4 slots XOR-swizzled by row, W n-contiguous
//    with rows padded by four floats; both keep the 16-byte LDS writes and the
//    MFMA fragment reads free of bank conflicts (the page pads its A tile to
//    17 for the same purpose).  Binary16 weights are widened to fp32 and the
//    SwiGLU combine silu(g) * u is applied to A on the way into LDS, so the
//    LDS tiles always hold the exact fp32 operands.
//  * Global loads are 16-byte (8-byte for four binary16 weights) buffer loads,
//    coalesced along the contiguous dimension.
//  * On gfx950 fp32 MFMA and VALU work do not overlap on a SIMD, so every
//    VALU cycle of staging is taken from the MFMAs: fp32 W is a plain copy,
//    W16 costs one conversion per element, A costs only the SwiGLU combine.
//  * Specialised pipeline: staging waves (loads, combine, LDS writes, one to
//    three K-stages of loads in flight) run beside compute waves (LDS reads
//    and MFMAs only) at a higher wave priority, over two LDS stages with one
//    barrier per stage (the page's "Çift Arabelleğe Alma").  Cooperative
//    configurations, where every wave does both, remain for comparison.
//  * Small output grids also split K across the compute waves of a
//    workgroup; their partial tiles are added through LDS in a fixed order.
//  * Workgroups are handed to the 8 XCDs round-robin; the tile order is
//    renumbered so that each XCD works on a contiguous, M-grouped range of
//    tiles and its private L2 sees reuse of both operands.
//  * Edges: rows >= M, columns >= N and k >= K are staged as zeros and never
//    read; stores are masked to i < M, j < N.
//  * The backward products give one operand transposed; it is staged in the
//    other operand's LDS layout (see the operand layouts below), so one
//    kernel template serves all of them.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "gemm_fwd.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct Params {
    const float *A;  // X, or GATE
    const float *U;  // UP (SwiGLU only)
    const void *W;
    const float *R;
    float *Y;
    // fused SwiGLU backward epilogue only: GATE and UP [M x N] in, d UP out
    // (d GATE goes to Y)
    const float *EG, *EU;
    float *Y2;
    int M, K, N;
    int tiles_m, tiles_n;
    int group_m;     // M-tiles per group in the tile order
    int kchunk;      // K range of one split (a multiple of BK) when K is split
    // split-K only (KS > 1), in the caller's workspace: KS partial tiles per
    // output tile (split s writes its partial of output element (i, j) at
    // ws[s * ws_stride + i * N + j]) and one arrival counter per output tile,
    // zero between calls
    float *ws;
    unsigned *cnt;
    int64_t ws_stride;
};

// Split-K.  When a configuration splits K over KS workgroups per output
// tile, each writes its fp32 partial tile into its own slot of the caller's
// workspace, then bumps the tile's counter; the last to arrive adds the KS
// slots in the fixed order 0..KS-1 (so results do not depend on arrival
// order), adds R, writes Y and resets the counter to zero.
constexpr int kSkMaxSplit = 8;

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// Slot permutation of a K-major LDS row of SL float4 slots: slot s of row r
// lives at s ^ swz<SL>(r).  A 16-byte fragment read covers 16 consecutive
// rows at one logical slot; measured with the bank-conflict counter, it takes
// the minimum 4 LDS cycles with the permutations below.
//  - 8-slot rows (128 bytes, so consecutive rows alternate between the two
//    halves of the 64 banks): r ^ (r >> 2) in 3 bits.
//  - 16 or more slots (every row starts on bank 0): the permutation must
//    spread 16 rows over 16 slots, so it takes 4 bits; the 3-bit one took
//    8 cycles per read here.  r ^ (r >> 2) in 4 bits is a bijection on each
//    aligned block of 16 rows.  For 32-slot rows it is taken of r mod 16, so
//    that it repeats every 16 rows and the fragments of one wave (rows 16
//    apart) share one address: with three fragments per wave that saved 6%
//    of a 16 x 48 x 128 kernel's time, while on 16-slot rows the full-row
//    form measured 1% faster.
template <int SL>
__device__ __forceinline__ int swz(int r) {
    if constexpr (SL >= 32) {
        const int b = r & 15;
        return b ^ (b >> 2);
    } else if constexpr (SL == 16) {
        return (r ^ (r >> 2)) & 15;
    } else {
        return (r ^ (r >> 2)) & 7;
    }
}

// silu(g) * u = g * u / (1 + exp(-g)), the sigmoid of "ffn_gelu_backward ve
// ffn_swiglu_backward — FFN Activation Backward" ("Türevler / SiLU'").  The
// page branches on the sign of g so that its exponential never overflows;
// here the overflow is harmless and dropping the branch saves three VALU
// operations: for g < -88.7 exp(-g) is +inf, its reciprocal 0, and the
// result a zero, the limit of the exact value (below 1e-36 in magnitude).
// Six VALU operations per element, two of them transcendental.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float t = __expf(-g);
    return (g * u) * __builtin_amdgcn_rcpf(1.0f + t);
}

// Block index -> (tile_m, tile_n).  Consecutive workgroup ids go to XCDs
// 0..7 in turn; renumber so that XCD x owns the contiguous range
// [x*q + min(x, r), ...) of the tile order, then walk that order in groups
// of group_m M-tiles (M fastest inside a group) for L2 reuse.
// With KS > 1 the KS workgroups of one tile are consecutive in that order
// (split fastest), so they also share an XCD.
template <int KS>
__device__ __forceinline__ void tile_coords(const Params &p, int &tm, int &tn, int &split) {
    const int nb = gridDim.x;
    const int b = blockIdx.x;
    const int q = nb >> 3, r = nb & 7, x = b & 7;
    const int tt = x * q + (x < r ? x : r) + (b >> 3);
    split = tt % KS;
    const int t = tt / KS;
    const int per_group = p.group_m * p.tiles_n;
    const int g = t / per_group;
    const int first_m = g * p.group_m;
    const int rows = min(p.tiles_m - first_m, p.group_m);
    const int in_g = t - g * per_group;
    tm = first_m + in_g % rows;
    tn = in_g / rows;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Buffer resource over [base, base + bytes): loads at an offset >= bytes
// return zeros without touching memory.  Masked elements (rows >= M, k >= K,
// columns >= N) are loaded at kOOB, which is past every resource's end, so
// the loads need no branches.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kOOB = (int)0x80000000u;

// The base and size are the same in every lane; readfirstlane states that to
// the compiler so the descriptor lives in scalar registers.
__device__ __forceinline__ Rsrc make_rsrc(const void *base, int bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    void *ub = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ f32x4 load_f32x4(Rsrc r, int off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

typedef unsigned int u32x4v __attribute__((vector_size(16)));

// 16-byte buffer load whose destination is LDS: lane l of the wave writes
// bytes [16 l, 16 l + 16) after `dst` (uniform across the wave), with zeros
// for an out-of-range offset.  The builtin exists only for the device pass.
__device__ __forceinline__ void load_f32x4_to_lds(Rsrc r, float *dst, int off) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
#else
    (void)r; (void)dst; (void)off;
#endif
}

// s_waitcnt for at most N outstanding vector memory operations (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their
// maxima, i.e. not waited for).
template <unsigned N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15u) | (7u << 4) | (15u << 8) | (((N >> 4) & 3u) << 14));
}


// Verification build (compiled with -DGEMM_SYNC_CHECK, a second library
// beside the shipping one): every barrier of the GEMM kernels first waits
// for all outstanding memory operations (s_waitcnt 0), the waits for
// LDS-destination loads wait for every load instead of all but the later
// stages' register loads, and the split-K exchange adds device-scope fences
// around the arrival count.  Same arithmetic in the same order, so its
// results must equal the shipping build's bit for bit; a difference would
// expose a hand-counted wait or an ordering that relies on timing.
#ifdef GEMM_SYNC_CHECK
constexpr bool kSyncCheck = true;
#else
constexpr bool kSyncCheck = false;
#endif

__device__ __forceinline__ void stage_barrier() {
    if constexpr (kSyncCheck) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Out-of-range stores (offset >= resource size) are dropped by the hardware.
__device__ __forceinline__ void store_f32x4(Rsrc r, int off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), r, off, 0, 0);
}

// Device-coherent 16-byte accesses (the sc1 cache policy, as used for
// agent-scope atomic loads and stores): written through to, and read from,
// the level shared by all XCDs.  Used only for split-K partial tiles.
constexpr int kCoherent = 16;
__device__ __forceinline__ void store_f32x4_coherent(Rsrc r, int off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ f32x4 load_f32x4_coherent(Rsrc r, int off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}

__device__ __forceinline__ f16x4 load_f16x4(Rsrc r, int voff) {
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}

// Tile configuration.  WM x WN x WK "compute" waves own the MFMAs (WM x WN
// wave tiles, K slices split over WK waves).  NP == 0: the same waves also
// stage the operands (cooperative pipeline).  NP > 0: NP further waves do
// all the staging (global loads, SwiGLU combine, f16 widening, LDS stores)
// while the compute waves only read LDS and issue MFMAs, so the two kinds of
// work overlap on every SIMD (specialised pipeline).  PF: register sets of
// staged K-stages per staging thread (1 to 5); loads run PF-1 stages ahead.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int WK_, int NP_, int PF_, int MINB_, int IL_ = 0,
          int KS_ = 1, int CIL_ = 0, int PRIO_ = 2, int DMA_ = 0, int WR_ = 0>
struct Tile {
    static constexpr bool CIL = CIL_ != 0;  // pipeline fragment reads one k-slice ahead of the MFMAs
    static constexpr int PRIO = PRIO_;      // wave priority of the staging waves
    // Specialised pipeline only: operands that need no arithmetic on the way
    // (bit 0: plain fp32 A, bit 1: fp32 W) go from memory straight into the
    // LDS stage by buffer loads with the LDS destination, bypassing VGPRs.
    static constexpr int DMA = DMA_;
    // Specialised pipeline, fp32 W in its natural layout only: WR > 0 keeps W
    // out of LDS.  Each compute wave loads the W fragments of its own k-slices
    // straight into a ring of WR slices of registers, WR - 1 slices ahead of
    // its MFMAs; the LDS stages hold A alone.  (Other instantiations of such a
    // tile stage W through LDS as usual.)
    static constexpr int WR = WR_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WM = WM_, WN = WN_, WK = WK_;
    static constexpr int NP = NP_, PF = PF_, MINB = MINB_;
    static constexpr bool IL = IL_ != 0;  // interleave staging loads with VALU/LDS work
    static constexpr int KS = KS_;        // workgroups sharing one output tile's K range
    static constexpr int NC = 64 * WM * WN * WK;        // compute threads
    static constexpr int NS = NP > 0 ? 64 * NP : NC;    // staging threads
    static constexpr int NT = NC + 64 * NP;             // block size
};

// Registers holding one K-stage of A (and UP) and W between its global load
// and its LDS store.  Each W item is four consecutive columns of one row.
template <int A_IT, int B_IT, bool SWIGLU, bool W16>
struct StageRegs {
    f32x4 a[A_IT > 0 ? A_IT : 1];
    f32x4 u[SWIGLU && A_IT > 0 ? A_IT : 1];
    typename std::conditional<W16, f16x4, f32x4>::type b[B_IT > 0 ? B_IT : 1];
};

// Operand layouts.  kOpNN: A [M x K] and B [K x N], both row-major (the
// forward products).  kOpNT: B is given as its transpose, [N x K] row-major
// (matmul_t, dX = dY W^T with the forward W [K x N]).  kOpTN: A is given as
// its transpose, [K x M] row-major (matmul_at, dW = X^T dY).  A transposed
// operand is staged the way the other operand's natural layout is: the LDS
// tile of an operand is always either contraction-contiguous (swizzled rows,
// one 16-byte read per MFMA fragment) or output-contiguous (padded rows, four
// reads per fragment), whichever its memory layout makes a plain copy.
constexpr int kOpNN = 0, kOpNT = 1, kOpTN = 2;

// Epilogues.  kEpiStore: Y = acc (+ R).  kEpiSwigluBwd: acc is the gradient
// dH of the SwiGLU activation H = silu(GATE) * UP, which is not stored;
// instead Y = dGATE = nan_guard(dH UP silu'(GATE)) and Y2 = dUP =
// nan_guard(dH silu(GATE)), with silu'(x) = s (1 + x (1 - s)), s the
// sign-branched sigmoid ("ffn_gelu_backward ve ffn_swiglu_backward",
// sections "Türevler" and "Satır Satır").
constexpr int kEpiStore = 0, kEpiSwigluBwd = 1;

__device__ __forceinline__ float nan_guard(float x) { return __builtin_isfinite(x) ? x : 0.0f; }

__device__ __forceinline__ void swiglu_bwd4(f32x4 dh, f32x4 g, f32x4 u, f32x4 &dg, f32x4 &du) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float x = g[c];
        const float e = __expf(-__builtin_fabsf(x));
        const float r = 1.0f / (1.0f + e);
        const float sg = x >= 0.0f ? r : e * r;
        dg[c] = nan_guard(dh[c] * u[c] * (sg * (1.0f + x * (1.0f - sg))));
        du[c] = nan_guard(dh[c] * (x * sg));
    }
}

template <class C, bool SWIGLU, bool W16, bool RESID, int OP = kOpNN, int EPI = kEpiStore>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_fwd_kernel(Params p) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK;
    constexpr int WM = C::WM, WN = C::WN, WK = C::WK;
    constexpr int NC = C::NC, NS = C::NS;
    constexpr bool SPEC = C::NP > 0;
    constexpr int SL = BK / 4;              // float4 slots per LDS row
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int CH = BK / 16;             // 16-wide k slices per stage
    constexpr bool AT = OP == kOpTN, BT = OP == kOpNT;
    static_assert(!(BT && W16), "a transposed B is fp32");
    static_assert(!(SWIGLU && OP == kOpNT), "the SwiGLU operand is A");
    constexpr int A_F4 = BM * SL;           // float4s of A per stage
    constexpr int MQ = BM / 4;              // transposed A: float4s per row of the tile
    constexpr int A_MB = BK * MQ;
    constexpr int A_ITEMS = AT ? A_MB : A_F4;
    constexpr int A_IT = (A_ITEMS + NS - 1) / NS;
    constexpr int NQ = BN / 4;              // float4s per W row in the tile
    constexpr int B_MB = BK * NQ;           // W items (row x 4 columns) per stage
    constexpr int B_F4 = BN * SL;           // transposed B: float4s per stage
    constexpr int B_ITEMS = BT ? B_F4 : B_MB;
    constexpr int B_IT = (B_ITEMS + NS - 1) / NS;
    constexpr int ASTR = BM + 4;            // padded LDS row of a transposed A tile (floats)
    constexpr int BSTR = BN + 4;            // padded LDS row of the W tile (floats)
    // W straight into the compute waves' registers (no W in LDS)
    constexpr bool WREG = C::WR > 0 && SPEC && !W16 && !BT;
    constexpr int A_LDS = AT ? BK * ASTR : BM * BK;  // floats of the A tile
    constexpr int B_LDS = WREG ? 0 : BT ? BN * BK : BK * BSTR;
    constexpr int STAGE = A_LDS + B_LDS;    // floats per LDS stage
    constexpr int CSTR = BN + 4;            // padded row of the output tile in LDS
    constexpr int CTILE = WK * BM * CSTR;   // floats for the output tile(s) in LDS
    static_assert(C::DMA == 0 || C::PF >= 2, "LDS-destination staging needs two register sets");
    constexpr int LDS_FLOATS = (2 * STAGE > CTILE) ? 2 * STAGE : CTILE;
    constexpr int WBYTES = W16 ? 2 : 4;
    static_assert(BK % 32 == 0, "swizzle needs at least 8 slots per row");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be MFMA tiles");
    static_assert(CH % WK == 0, "K slices must split evenly over waves");

    __shared__ __attribute__((aligned(16))) float lds[LDS_FLOATS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform role: compute waves first, then staging-only waves
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool computes = wave < WM * WN * WK;
    const bool stages = SPEC ? !computes : true;
    const int stid = SPEC ? tid - NC : tid;  // index among staging threads
    const int wk = wave % WK;
    const int wmn = wave / WK;
    const int wm = wmn / WN, wn = wmn % WN;

    constexpr int KS = C::KS;
    static_assert(KS >= 1 && KS <= kSkMaxSplit, "split count");
    int tm, tn, split;
    tile_coords<KS>(p, tm, tn, split);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, K = p.K, N = p.N;
    // this workgroup's K range [kbeg, kend)
    const int kbeg = KS > 1 ? split * p.kchunk : 0;
    const int kend = KS > 1 ? min(K, kbeg + p.kchunk) : K;

    // A (and UP) resources span the tile's valid rows, so rows >= M read as 0.
    const int rows_valid = min(BM, M - m0);
    // The A (and UP) resources of a stage start at column k0 of the tile's
    // first row and end with its last valid row, so rows >= M read as 0.
    // A transposed operand starts at column m0 (A) or row n0 (B) instead.
    const float *Abase = AT ? p.A + m0 : p.A + (size_t)m0 * K;
    const float *Ubase = SWIGLU ? (AT ? p.U + m0 : p.U + (size_t)m0 * K) : Abase;
    const int abytes = AT ? 0 : rows_valid * K * 4;
    const char *Wbase = static_cast<const char *>(p.W) + (BT ? (size_t)n0 * K * 4 : (size_t)n0 * WBYTES);
    const int bbytes = BT ? min(BN, N - n0) * K * 4 : 0;   // transposed B: the tile's valid rows

    // Per-thread staging coordinates (fixed over the K loop).
    int a_off[A_IT], a_gk[A_IT];
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
        const int f = stid + i * NS;
        if constexpr (AT) {
            // rows k of the stage, 4 columns each; columns >= M and padding
            // items read out of range, rows past the K range fall outside
            // the stage's resource
            const int k = f / MQ, mq = f % MQ;
            const bool live = (A_IT * NS == A_MB || f < A_MB) && (m0 + mq * 4 < M);
            a_off[i] = live ? (k * M + mq * 4) * 4 : kOOB;
            a_gk[i] = 0;
        } else {
            const int row = f / SL, slot = f % SL;
            a_gk[i] = (A_IT * NS == A_F4 || f < A_F4) ? slot * 4 : K;  // out-of-range f: always masked
            a_off[i] = (row * K + slot * 4) * 4;
        }
    }
    // W items: consecutive staging threads take consecutive 4-column groups
    // of a row, so each load instruction reads contiguous memory.  Rows past
    // the K range fall outside the stage's W resource, so only items outside
    // the tile (columns >= N, padding items) need the kOOB offset.
    int b_off[B_IT], b_gk[BT ? B_IT : 1];
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
        const int mb = stid + i * NS;
        if constexpr (BT) {
            // as A: rows n of the tile, 4 consecutive k each; rows >= N fall
            // outside the resource, k past the K range is masked per stage
            const int row = mb / SL, slot = mb % SL;
            b_gk[i] = (B_IT * NS == B_F4 || mb < B_F4) ? slot * 4 : K;
            b_off[i] = (row * K + slot * 4) * 4;
        } else {
            const int k = mb / NQ, nq = mb % NQ;
            const bool live = (B_IT * NS == B_MB || mb < B_MB) && (n0 + nq * 4 < N);
            b_off[i] = live ? (k * N + nq * 4) * WBYTES : kOOB;
        }
    }

    // Operands staged by LDS-destination loads, and the register items left.
    constexpr bool DMA_A = (C::DMA & 1) && !SWIGLU && SPEC && !AT;
    constexpr bool DMA_W = (C::DMA & 2) && !W16 && SPEC && !BT && !WREG;
    constexpr int A_RIT = DMA_A ? 0 : A_IT;
    constexpr int B_RIT = DMA_W || WREG ? 0 : B_IT;
    constexpr int REG_LOADS = A_RIT * (SWIGLU ? 2 : 1) + B_RIT;  // register loads per stage
    typedef StageRegs<A_RIT, B_RIT, SWIGLU, W16> Regs;

    // One LDS-destination load moves 64 float4 slots (1 KiB) into a
    // contiguous LDS range, lane l into slot l; each lane picks the global
    // float4 that belongs in its slot, so the swizzled A layout and the
    // padded W rows come out as the register path writes them (pad slots
    // and masked elements are fetched out of range and land as zeros).
    constexpr int W_SPR = NQ + 1;                 // float4 slots per padded W row
    constexpr int A_CH = A_F4 / 64;               // 64-slot chunks per stage
    constexpr int W_CH = BK * W_SPR / 64;
    static_assert(!DMA_A || A_F4 % 64 == 0, "A tile must be whole 64-slot chunks");
    static_assert(!DMA_W || (BK * W_SPR) % 64 == 0, "padded W tile must be whole 64-slot chunks");
    constexpr int NPW = SPEC ? C::NP : 1;
    constexpr int A_DIT = DMA_A ? (A_CH + NPW - 1) / NPW : 0;  // chunks per staging wave
    constexpr int W_DIT = DMA_W ? (W_CH + NPW - 1) / NPW : 0;
    const int pw = SPEC ? wave - NC / 64 : 0;     // staging wave index (uniform)
    int ad_off[A_DIT > 0 ? A_DIT : 1], ad_gk[A_DIT > 0 ? A_DIT : 1];
#pragma unroll
    for (int j = 0; j < A_DIT; ++j) {
        const int q = (pw + j * NPW) * 64 + lane;
        const int row = q / SL, logical = (q % SL) ^ swz<SL>(row);
        ad_gk[j] = logical * 4;
        ad_off[j] = (row * K + logical * 4) * 4;
    }
    int wd_off[W_DIT > 0 ? W_DIT : 1];
#pragma unroll
    for (int j = 0; j < W_DIT; ++j) {
        const int q = (pw + j * NPW) * 64 + lane;
        const int k = q / W_SPR, s4 = q % W_SPR;
        const bool live = s4 < NQ && n0 + s4 * 4 < N;
        wd_off[j] = live ? (k * N + s4 * 4) * 4 : kOOB;
    }
    auto dma_stage = [&](int buf, int k0) {
        float *S = lds + buf * STAGE;
        const int krem = kend - k0;
        if constexpr (DMA_A) {
            const int arem = abytes - k0 * 4;
            const Rsrc rA = make_rsrc(Abase + k0, arem > 0 ? arem : 0);
            // a stage wholly inside the K range needs no per-item check
            // (krem is uniform, so this is a scalar branch)
            if (krem >= BK) {
#pragma unroll
                for (int j = 0; j < A_DIT; ++j) {
                    const int c = pw + j * NPW;
                    if (A_CH % NPW != 0 && c >= A_CH) break;
                    load_f32x4_to_lds(rA, S + c * 256, ad_off[j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < A_DIT; ++j) {
                    const int c = pw + j * NPW;
                    if (A_CH % NPW != 0 && c >= A_CH) break;
                    const int off = ad_gk[j] < krem ? ad_off[j] : kOOB;
                    load_f32x4_to_lds(rA, S + c * 256, off);
                }
            }
        }
        if constexpr (DMA_W) {
            const Rsrc rW = make_rsrc(Wbase + (size_t)k0 * N * WBYTES,
                                      krem > 0 ? min(krem, BK) * N * WBYTES : 0);
#pragma unroll
            for (int j = 0; j < W_DIT; ++j) {
                const int c = pw + j * NPW;
                if (W_CH % NPW != 0 && c >= W_CH) break;
                load_f32x4_to_lds(rW, S + A_LDS + c * 256, wd_off[j]);
            }
        }
        // keep the register loads that follow behind these in issue order, so
        // that a vmcnt of the later ones' count covers them
        __builtin_amdgcn_sched_barrier(0);
    };
    // Wait until at most the register loads of the last n stages are
    // outstanding, so every LDS-destination load issued before them landed.
    auto dma_wait = [&](auto n) {
        if constexpr (DMA_A || DMA_W) wait_vmcnt<kSyncCheck ? 0u : decltype(n)::value * REG_LOADS>();
    };

    auto load_stage = [&](Regs &r, int k0) {
        // per stage only scalar work moves the resources; per item the A
        // column is checked against the K range (one compare, one select)
        const int krem = kend - k0;
        if constexpr (AT) {
            // rows k0 .. k0+BK-1 of the transposed A, from column m0
            const int tbytes = krem > 0 ? min(krem, BK) * M * 4 : 0;
            const Rsrc rA = make_rsrc(Abase + (size_t)k0 * M, tbytes);
            const Rsrc rU = SWIGLU ? make_rsrc(Ubase + (size_t)k0 * M, tbytes) : rA;
#pragma unroll
            for (int i = 0; i < A_RIT; ++i) {
                r.a[i] = load_f32x4(rA, a_off[i]);
                if constexpr (SWIGLU) r.u[i] = load_f32x4(rU, a_off[i]);
            }
        } else {
            const int arem = abytes - k0 * 4;
            const Rsrc rA = make_rsrc(Abase + k0, arem > 0 ? arem : 0);
            const Rsrc rU = SWIGLU ? make_rsrc(Ubase + k0, arem > 0 ? arem : 0) : rA;
#pragma unroll
            for (int i = 0; i < A_RIT; ++i) {
                const int off = a_gk[i] < krem ? a_off[i] : kOOB;
                r.a[i] = load_f32x4(rA, off);
                if constexpr (SWIGLU) r.u[i] = load_f32x4(rU, off);
            }
        }
        // W rows k0 .. k0+BK-1 from a resource based at row k0 that ends at
        // the K range, so offsets stay 32-bit whatever K * N is and rows past
        // the range read as 0.
        if constexpr (BT) {
            // the tile's valid rows of the transposed B, from column k0
            const int brem = bbytes - k0 * 4;
            const Rsrc rB = make_rsrc(reinterpret_cast<const float *>(Wbase) + k0, brem > 0 ? brem : 0);
#pragma unroll
            for (int i = 0; i < B_RIT; ++i) r.b[i] = load_f32x4(rB, b_gk[i] < krem ? b_off[i] : kOOB);
        } else {
            const Rsrc rW = make_rsrc(Wbase + (size_t)k0 * N * WBYTES,
                                      krem > 0 ? min(krem, BK) * N * WBYTES : 0);
#pragma unroll
            for (int i = 0; i < B_RIT; ++i) {
                if constexpr (W16) r.b[i] = load_f16x4(rW, b_off[i]);
                else r.b[i] = load_f32x4(rW, b_off[i]);
            }
        }
    };

    auto store_stage = [&](const Regs &r, int buf) {
        float *As = lds + buf * STAGE;
        float *Bs = As + A_LDS;
#pragma unroll
        for (int i = 0; i < A_RIT; ++i) {
            const int f = stid + i * NS;
            if (A_IT * NS != A_ITEMS && f >= A_ITEMS) continue;
            f32x4 v = r.a[i];
            if constexpr (SWIGLU) {
                v.x = silu_mul(v.x, r.u[i].x);
                v.y = silu_mul(v.y, r.u[i].y);
                v.z = silu_mul(v.z, r.u[i].z);
                v.w = silu_mul(v.w, r.u[i].w);
            }
            if constexpr (AT) {
                const int k = f / MQ, mq = f % MQ;
                *reinterpret_cast<f32x4 *>(As + k * ASTR + mq * 4) = v;
            } else {
                const int row = f / SL, slot = f % SL;
                *reinterpret_cast<f32x4 *>(As + (row * SL + (slot ^ swz<SL>(row))) * 4) = v;
            }
        }
#pragma unroll
        for (int i = 0; i < B_RIT; ++i) {
            const int mb = stid + i * NS;
            if (B_IT * NS != B_ITEMS && mb >= B_ITEMS) continue;
            if constexpr (BT) {
                const int row = mb / SL, slot = mb % SL;
                *reinterpret_cast<f32x4 *>(Bs + (row * SL + (slot ^ swz<SL>(row))) * 4) = r.b[i];
                continue;
            }
            const int k = mb / NQ, nq = mb % NQ;
            f32x4 t;
            if constexpr (W16) {
                t = f32x4{static_cast<float>(r.b[i][0]), static_cast<float>(r.b[i][1]),
                          static_cast<float>(r.b[i][2]), static_cast<float>(r.b[i][3])};
            } else {
                t = r.b[i];
            }
            *reinterpret_cast<f32x4 *>(Bs + k * BSTR + nq * 4) = t;
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15, q4 = lane >> 4;

    // W in registers (WREG).  For row 4*q4 + t of a 16-row k-slice, lane
    // (q4, r16) holds TN columns of its wave tile: WG groups of WV
    // consecutive columns, one load each, group g starting at column
    // 16*WV*g + WV*r16 of the wave tile.  The wave's MFMA tile j takes
    // column WV*r16 + j % WV of group j / WV, so the accumulators hold the
    // wave tile's columns in a permuted order, undone where the epilogue
    // parks them in LDS.  Groups never straddle N (N and WV*r16 are
    // multiples of WV), so a group is either loaded whole or masked whole.
    constexpr int WV = TN % 4 == 0 ? 4 : TN % 2 == 0 ? 2 : 1;
    constexpr int WG = TN / WV;
    constexpr int NCH = CH / WK;            // k-slices per stage of one wave
    constexpr int WR = WREG ? C::WR : 1;
    static_assert(!WREG || (WR >= 2 && NCH % WR == 0), "W ring slots must divide a stage's slices");
    int wr_off[WREG ? 4 : 1][WREG ? WG : 1];
    float wring[WR][WREG ? 4 : 1][WREG ? TN : 1];
    if constexpr (WREG) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int g = 0; g < WG; ++g) {
                const int col = wn * WTN + g * 16 * WV + WV * r16;
                wr_off[t][g] = n0 + col < N ? ((4 * q4 + t) * N + col) * 4 : kOOB;
            }
    }
    // The W fragments of the 16-row slice starting at row kk, from a resource
    // that holds the slice's rows inside the K range (none past it).
    // W's tile origin as a wave-uniform 64-bit value, so that the per-slice
    // resource base is scalar arithmetic (readfirstlane returns a signed
    // int: each half goes through uint32_t before it is widened)
    const uint32_t wtile_lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uint64_t>(Wbase)));
    const uint32_t wtile_hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uint64_t>(Wbase) >> 32));
    const uint64_t wtile = (static_cast<uint64_t>(wtile_hi) << 32) | wtile_lo;
    auto wload = [&](float (&d)[WREG ? 4 : 1][WREG ? TN : 1], int kk) {
        if constexpr (WREG) {
            const int rem = kend - kk;
            const Rsrc rW = make_rsrc(reinterpret_cast<const void *>(wtile + (uint64_t)(uint32_t)kk * (uint32_t)(N * 4)),
                                      rem > 0 ? min(rem, 16) * N * 4 : 0);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int g = 0; g < WG; ++g) {
                    if constexpr (WV == 4) {
                        const f32x4 v = load_f32x4(rW, wr_off[t][g]);
#pragma unroll
                        for (int v4 = 0; v4 < 4; ++v4) d[t][g * 4 + v4] = v[v4];
                    } else if constexpr (WV == 2) {
                        const f32x2 v = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rW, wr_off[t][g], 0, 0));
                        d[t][g * 2] = v[0];
                        d[t][g * 2 + 1] = v[1];
                    } else {
                        d[t][g] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rW, wr_off[t][g], 0, 0));
                    }
                }
        }
    };

    auto compute_stage = [&](int buf, int k0) {
        const float *As = lds + buf * STAGE;
        const float *Bs = As + A_LDS;
        if constexpr (WREG) {
            (void)Bs;
            // The A fragments of slice l + 1 are read while slice l is
            // multiplied; the W loads of slice l + WR - 1 go out between the
            // MFMAs of slice l.  Each slice is its own scheduling region, so
            // the compiler can neither sink those loads to their use nor
            // hoist the next slice's reads above them.
            auto read_a = [&](f32x4 (&af)[TM], int c) {
                const int slot = c * 4 + q4;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if constexpr (AT) {
                        const float *a = As + (c * 16 + q4 * 4) * ASTR + wm * WTM + i * 16 + r16;
                        af[i] = f32x4{a[0], a[ASTR], a[2 * ASTR], a[3 * ASTR]};
                    } else {
                        const int row = wm * WTM + i * 16 + r16;
                        af[i] = *reinterpret_cast<const f32x4 *>(As + (row * SL + (slot ^ swz<SL>(row))) * 4);
                    }
                }
            };
            constexpr int DS = AT ? 2 * TM : TM;  // LDS reads per slice
            constexpr int NL = 4 * WG;             // W loads per slice
            constexpr int MF = 4 * TM * TN;        // MFMAs per slice
            constexpr int PER = MF / NL > 0 ? MF / NL : 1;
            f32x4 afc[TM], afn[TM];
            read_a(afc, wk);
#pragma unroll
            for (int l = 0; l < NCH; ++l) {
                if (l + 1 < NCH) read_a(afn, wk + (l + 1) * WK);
                // slice l + WR - 1 (of this stage or the next) into the ring
                // slot that slice l - 1 used
                const int la = l + WR - 1;
                wload(wring[la % WR], k0 + (la < NCH ? (wk + la * WK) * 16 : BK + (wk + (la - NCH) * WK) * 16));
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(afc[i][t], wring[l % WR][t][j], acc[i][j], 0, 0, 0);
                if (l + 1 < NCH) __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
#pragma unroll
                for (int x = 0; x < NL; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
                }
                if constexpr (MF > NL * PER) __builtin_amdgcn_sched_group_barrier(0x008, MF - NL * PER, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TM; ++i) afc[i] = afn[i];
            }
            return;
        }
#pragma unroll
        for (int c = wk; c < CH; c += WK) {
            const int slot = c * 4 + q4;
            f32x4 af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if constexpr (AT) {
                    const float *a = As + (c * 16 + q4 * 4) * ASTR + wm * WTM + i * 16 + r16;
                    af[i] = f32x4{a[0], a[ASTR], a[2 * ASTR], a[3 * ASTR]};
                } else {
                    const int row = wm * WTM + i * 16 + r16;
                    af[i] = *reinterpret_cast<const f32x4 *>(As + (row * SL + (slot ^ swz<SL>(row))) * 4);
                }
            }
            // W is N-major in LDS: the four k of a lane are four rows; the row
            // padding puts rows k and k+4 sixteen banks apart.
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (BT) {
                    const int row = wn * WTN + j * 16 + r16;
                    bf[j] = *reinterpret_cast<const f32x4 *>(Bs + (row * SL + (slot ^ swz<SL>(row))) * 4);
                } else {
                    const float *b = Bs + (c * 16 + q4 * 4) * BSTR + wn * WTN + j * 16 + r16;
                    bf[j] = f32x4{b[0], b[BSTR], b[2 * BSTR], b[3 * BSTR]};
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][t], bf[j][t], acc[i][j], 0, 0, 0);
        }
        if constexpr (C::CIL && !WREG) {
            // Scheduling hint: read all fragments of the first k-slice, then
            // spread each later slice's reads over the MFMAs of the slice
            // before it, so LDS latency hides behind matrix work instead of
            // stalling in front of every few MFMAs.
            // b128 per contraction-contiguous fragment, two read2_b32 per other
            constexpr int DS = (AT ? 2 * TM : TM) + (BT ? TN : 2 * TN);
            constexpr int MF = 4 * TM * TN;
            constexpr int PER = (MF + DS - 1) / DS;
            __builtin_amdgcn_sched_group_barrier(0x100, DS, 0);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (c + 1 < NCH) {
#pragma unroll
                    for (int d = 0; d < DS; ++d) {
                        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                } else {
                    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
                }
            }
        }
    };

    // Scheduling hint for a staging step (loads of a later stage, then the
    // combine and LDS stores of the next one): alternate one global load with
    // a share of the VALU work and one LDS store, so the address unit drains
    // while the VALU works instead of stalling the wave at issue.
    auto interleave_hint = [&]() {
        if constexpr (C::IL) {
            constexpr int NLOAD = A_IT * (SWIGLU ? 2 : 1) + (WREG ? 0 : B_IT);
            constexpr int NVALU = (SWIGLU ? 24 * A_IT : 0) + (W16 ? 4 * B_IT : 0) + 2 * (A_IT + (WREG ? 0 : B_IT));
            constexpr int PER = (NVALU + NLOAD - 1) / NLOAD;
#pragma unroll
            for (int i = 0; i < NLOAD; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // global load
                __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);  // VALU
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);    // LDS store
            }
        }
    };

    // K loop over nstages stages of BK, LDS double-buffered, one barrier per
    // stage.  Loads past K are issued at kOOB and return zeros, so no stage
    // needs a branch on its position.
    //  PF == 2: two stages of loads in flight per staging thread: while stage
    //   s is multiplied out of one LDS buffer, stage s+1 waits in registers
    //   for the other buffer and stage s+2 is being fetched.
    //  PF == 1: the loads of stage s+1 overlap the MFMAs of stage s.
    const int nstages = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    if constexpr (SPEC) {
        // Staging waves run their own loop, one stage ahead of the compute
        // waves, and meet them at the same barriers (equal counts on both
        // sides, including the K-split reduction's).  Keeping the two loops
        // apart lets the staging registers and the accumulators share VGPRs.
        if (stages) {
            // Staging waves outrank the compute wave of their SIMD, so their
            // short VALU bursts slot in between MFMAs as soon as their data
            // lands, instead of queueing behind a whole stage of MFMAs and
            // holding the next barrier back.
            __builtin_amdgcn_s_setprio(C::PRIO);
            if (nstages > 0) {
                if constexpr (C::PF >= 3 || DMA_A || DMA_W) {
                    // PF register sets, stage t in set t % PF: each step
                    // first issues the loads of stage s+PF into the set just
                    // stored, then combines and stores stage s+1, so the
                    // address unit drains while the VALU works and every
                    // load has PF-1 steps to land.  LDS-destination loads of
                    // stage s+1 go out first in the step (their buffer is
                    // free since the last barrier) and are waited for just
                    // before the barrier.
                    constexpr int PF = C::PF;
                    Regs r[PF];
                    dma_stage(0, kbeg);
#pragma unroll
                    for (int j = 0; j < PF; ++j) load_stage(r[j], kbeg + j * BK);
                    store_stage(r[0], 0);
                    dma_wait(std::integral_constant<unsigned, PF - 1>{});
                    stage_barrier();
                    int s = 0;
                    for (; s + PF <= nstages; s += PF) {
#pragma unroll
                        for (int j = 0; j < PF; ++j) {
                            dma_stage((s + j + 1) & 1, kbeg + (s + j + 1) * BK);
                            load_stage(r[j], kbeg + (s + j + PF) * BK);
                            store_stage(r[(j + 1) % PF], (s + j + 1) & 1);
                            interleave_hint();
                            dma_wait(std::integral_constant<unsigned, 1>{});
                            stage_barrier();
                        }
                    }
#pragma unroll
                    for (int j = 0; j + 1 < PF; ++j) {
                        if (s + j < nstages) {
                            dma_stage((s + j + 1) & 1, kbeg + (s + j + 1) * BK);
                            store_stage(r[(j + 1) % PF], (s + j + 1) & 1);
                            dma_wait(std::integral_constant<unsigned, 0>{});
                            stage_barrier();
                        }
                    }
                } else if constexpr (C::PF == 2) {
                    Regs r0, r1;
                    load_stage(r0, kbeg + 0);
                    load_stage(r1, kbeg + BK);
                    store_stage(r0, 0);
                    load_stage(r0, kbeg + 2 * BK);
                    stage_barrier();
                    for (int s = 0;; s += 2) {
                        store_stage(r1, 1);
                        load_stage(r1, kbeg + (s + 3) * BK);
                        stage_barrier();
                        if (s + 1 >= nstages) break;
                        store_stage(r0, 0);
                        load_stage(r0, kbeg + (s + 4) * BK);
                        stage_barrier();
                        if (s + 2 >= nstages) break;
                    }
                } else {
                    Regs r0;
                    load_stage(r0, kbeg + 0);
                    store_stage(r0, 0);
                    load_stage(r0, kbeg + BK);
                    stage_barrier();
                    for (int s = 0;; ++s) {
                        store_stage(r0, (s + 1) & 1);
                        load_stage(r0, kbeg + (s + 2) * BK);
                        stage_barrier();
                        if (s + 1 >= nstages) break;
                    }
                }
            }
            stage_barrier();  // the epilogue's barrier
            if constexpr (KS > 1) {
                stage_barrier();  // partials stored
                stage_barrier();  // arrival counted
            }
            return;
        }
        if (nstages > 0) {
            if constexpr (WREG) {
#pragma unroll
                for (int l = 0; l + 1 < WR; ++l) wload(wring[l], kbeg + (wk + l * WK) * 16);
            }
            stage_barrier();
            for (int s = 0;; ++s) {
                compute_stage(s & 1, kbeg + s * BK);
                stage_barrier();
                if (s + 1 >= nstages) break;
            }
            // the ring's last loads (past the K range, so zeros) land before
            // their registers are reused
            if constexpr (WREG) wait_vmcnt<0>();
        }
    } else if (nstages > 0) {
        if constexpr (C::PF == 2) {
            Regs r0, r1;
            load_stage(r0, kbeg + 0);
            load_stage(r1, kbeg + BK);
            store_stage(r0, 0);
            stage_barrier();
            for (int s = 0;; s += 2) {
                load_stage(r0, kbeg + (s + 2) * BK);
                compute_stage(0, 0);
                store_stage(r1, 1);
                stage_barrier();
                if (s + 1 >= nstages) break;
                load_stage(r1, kbeg + (s + 3) * BK);
                compute_stage(1, 0);
                store_stage(r0, 0);
                stage_barrier();
                if (s + 2 >= nstages) break;
            }
        } else {
            Regs r0;
            load_stage(r0, kbeg + 0);
            store_stage(r0, 0);
            stage_barrier();
            for (int s = 0;; ++s) {
                load_stage(r0, kbeg + (s + 1) * BK);
                compute_stage(s & 1, 0);
                if (s + 1 >= nstages) break;
                store_stage(r0, (s + 1) & 1);
                stage_barrier();
            }
            // the last stage was read without a closing barrier
            stage_barrier();
        }
    }

    // Epilogue through LDS (every K loop above ends with a barrier after its
    // last read of the stages).  Each compute wave parks its accumulators in
    // a padded row-major copy of the output tile, one copy per K-slice wave;
    // then every compute thread takes whole float4s of the tile, adds the
    // K-slice copies in the fixed order 0, 1, ..., WK-1, adds R, and stores
    // Y with 16-byte buffer accesses.  Lane (q4, r16) of a 16x16 MFMA tile
    // holds rows 4*q4 .. 4*q4+3 of column r16.
    if (computes) {
        float *Ct = lds + wk * BM * CSTR;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Ct[(wm * WTM + i * 16 + q4 * 4 + r) * CSTR + wn * WTN +
                       (WREG ? (j / WV) * 16 * WV + WV * r16 + j % WV : j * 16 + r16)] = acc[i][j][r];
    }
    stage_barrier();

    const size_t tile_off = (size_t)m0 * N + n0;
    // The last step of the epilogue for four consecutive outputs at byte
    // offset `off` of the tile (kOOB for masked items): store them (plus R),
    // or turn them into the two SwiGLU gradients.
    auto make_finish = [&](int ybytes) {
        const Rsrc rY = make_rsrc(p.Y + tile_off, ybytes);
        const Rsrc rR = RESID ? make_rsrc(p.R + tile_off, ybytes) : rY;
        const Rsrc rG = EPI == kEpiSwigluBwd ? make_rsrc(p.EG + tile_off, ybytes) : rY;
        const Rsrc rU = EPI == kEpiSwigluBwd ? make_rsrc(p.EU + tile_off, ybytes) : rY;
        const Rsrc rY2 = EPI == kEpiSwigluBwd ? make_rsrc(p.Y2 + tile_off, ybytes) : rY;
        return [=](f32x4 v, int off) {
            if constexpr (EPI == kEpiSwigluBwd) {
                f32x4 dg, du;
                swiglu_bwd4(v, load_f32x4(rG, off), load_f32x4(rU, off), dg, du);
                store_f32x4(rY, off, dg);
                store_f32x4(rY2, off, du);
            } else {
                if constexpr (RESID) v += load_f32x4(rR, off);
                store_f32x4(rY, off, v);
            }
        };
    };
    constexpr int Q = BN / 4;
    constexpr int ITEMS = BM * Q;
    if constexpr (KS > 1) {
        // Publish this split's partial tile, then count the arrival.
        __shared__ int sk_last;
        const int tile_id = tm * p.tiles_n + tn;
        // the tile's valid rows span rows_valid * N elements of a slot
        const int pbytes = rows_valid * N * 4;
        if (computes) {
            const Rsrc rP = make_rsrc(p.ws + split * p.ws_stride + tile_off, pbytes);
#pragma unroll
            for (int it = 0; it < (ITEMS + NC - 1) / NC; ++it) {
                const int idx = tid + it * NC;
                if (ITEMS % NC != 0 && idx >= ITEMS) break;
                const int row = idx / Q, c4 = idx % Q;
                f32x4 v = *reinterpret_cast<const f32x4 *>(lds + row * CSTR + c4 * 4);
#pragma unroll
                for (int w = 1; w < WK; ++w)
                    v += *reinterpret_cast<const f32x4 *>(lds + (w * BM + row) * CSTR + c4 * 4);
                const bool ok = (m0 + row < M) && (n0 + c4 * 4 < N);
                store_f32x4_coherent(rP, ok ? (row * N + c4 * 4) * 4 : kOOB, v);
            }
        }
        // Every thread's coherent partial stores have completed before the
        // barrier, so they are visible device-wide before the arrival count
        // moves.  (A device-scope fence would write back and invalidate the
        // whole L2 of the XCD instead.)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        if constexpr (kSyncCheck) __threadfence();
        stage_barrier();
        if (tid == 0)
            sk_last = __hip_atomic_fetch_add(p.cnt + tile_id, 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(KS - 1);
        stage_barrier();
        if (!sk_last || !computes) return;
        if constexpr (kSyncCheck) __threadfence();
        if (tid == 0)
            __hip_atomic_store(p.cnt + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int ybytes = rows_valid * N * 4;
        const auto finish = make_finish(ybytes);
#pragma unroll
        for (int it = 0; it < (ITEMS + NC - 1) / NC; ++it) {
            const int idx = tid + it * NC;
            if (ITEMS % NC != 0 && idx >= ITEMS) break;
            const int row = idx / Q, c4 = idx % Q;
            const bool ok = (m0 + row < M) && (n0 + c4 * 4 < N);
            const int off = ok ? (row * N + c4 * 4) * 4 : kOOB;
            // this split's own partial is still in LDS; the others come from
            // the workspace.  Summation order 0..KS-1 whatever arrived last.
            f32x4 own = *reinterpret_cast<const f32x4 *>(lds + row * CSTR + c4 * 4);
#pragma unroll
            for (int w = 1; w < WK; ++w)
                own += *reinterpret_cast<const f32x4 *>(lds + (w * BM + row) * CSTR + c4 * 4);
            f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sp = 0; sp < KS; ++sp) {
                if (sp == split) {
                    v += own;
                } else {
                    v += load_f32x4_coherent(make_rsrc(p.ws + sp * p.ws_stride + tile_off, pbytes), off);
                }
            }
            finish(v, off);
        }
        return;
    }
    if (!computes) return;

    // The tile's valid rows span rows_valid * N elements from its origin
    // (under 2^30 bytes by the shape limits); masked items use kOOB.
    const int ybytes = rows_valid * N * 4;
    const auto finish = make_finish(ybytes);
#pragma unroll
    for (int it = 0; it < (ITEMS + NC - 1) / NC; ++it) {
        const int idx = tid + it * NC;
        if (ITEMS % NC != 0 && idx >= ITEMS) break;
        const int row = idx / Q, c4 = idx % Q;
        f32x4 v = *reinterpret_cast<const f32x4 *>(lds + row * CSTR + c4 * 4);
#pragma unroll
        for (int w = 1; w < WK; ++w)
            v += *reinterpret_cast<const f32x4 *>(lds + (w * BM + row) * CSTR + c4 * 4);
        const bool ok = (m0 + row < M) && (n0 + c4 * 4 < N);
        const int off = ok ? (row * N + c4 * 4) * 4 : kOOB;
        finish(v, off);
    }
}

// Y = R (or 0) when K == 0: the contraction is empty.
__global__ void fill_k0_kernel(const float *R, float *Y, int64_t count) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) Y[i] = R ? R[i] : 0.0f;
}

// ---------------------------------------------------------------------------
// configuration table
// ---------------------------------------------------------------------------

typedef void (*KernelFn)(Params);

struct ConfigEntry {
    const char *name;
    int bm, bn, bk, nt, ks;
    KernelFn fn[2][2][2];  // [swiglu][w16][resid]
};

// A tile that keeps W in registers (WR > 0) exists for fp32 W only: its
// f16 W slots are empty and such a call gives GEMM_ERR_CONFIG.
template <class C, bool SWIGLU, bool W16, bool RESID>
constexpr KernelFn fwd_fn() {
    if constexpr (W16 && C::WR > 0) return nullptr;
    else return gemm_fwd_kernel<C, SWIGLU, W16, RESID>;
}

template <class C>
constexpr ConfigEntry make_entry(const char *name) {
    return ConfigEntry{name, C::BM, C::BN, C::BK, C::NT, C::KS,
                       {{{fwd_fn<C, false, false, false>(), fwd_fn<C, false, false, true>()},
                         {fwd_fn<C, false, true, false>(), fwd_fn<C, false, true, true>()}},
                        {{fwd_fn<C, true, false, false>(), fwd_fn<C, true, false, true>()},
                         {fwd_fn<C, true, true, false>(), fwd_fn<C, true, true, true>()}}}};
}

// Tile<BM, BN, BK, WM, WN, WK, NP, PF, MINB, IL, KS, CIL, PRIO, DMA, WR>: the
// tiles the library's own forward choice takes (select_config), then one of
// each other kind of pipeline, so that every code path stays built and
// tested.
const ConfigEntry kConfigs[] = {
    make_entry<Tile<128, 128, 32, 2, 2, 1, 4, 3, 1, 1, 1, 0, 2, 1>>("128x128x32_w2x2_sp4_pf3_il_dA"),
    make_entry<Tile<64, 384, 32, 1, 4, 1, 8, 4, 1, 1>>("64x384x32_w1x4_sp8_pf4_il"),
    make_entry<Tile<128, 192, 32, 2, 2, 1, 8, 4, 1, 1>>("128x192x32_w2x2_sp8_pf4_il"),
    make_entry<Tile<128, 64, 32, 2, 2, 1, 4, 3, 1, 1, 1, 0, 2, 1>>("128x64x32_w2x2_sp4_pf3_il_dA"),
    make_entry<Tile<64, 64, 64, 2, 2, 1, 4, 2, 1, 0, 1, 0, 2, 3>>("64x64x64_w2x2_sp4_dAW"),
    // the same tile with K split over two workgroups (one whole round of
    // tiles over a long contraction)
    make_entry<Tile<64, 64, 64, 2, 2, 1, 4, 2, 1, 0, 2, 0, 2, 3>>("64x64x64_w2x2_sp4_ks2_dAW"),
    make_entry<Tile<128, 48, 32, 2, 1, 2, 4, 3, 1, 1, 1, 0, 2, 1>>("128x48x32_w2x1_k2_sp4_pf3_il_dA"),
    make_entry<Tile<64, 48, 64, 2, 1, 2, 4, 3, 1, 1, 1, 0, 2, 1>>("64x48x64_w2x1_k2_sp4_pf3_il_dA"),
    make_entry<Tile<32, 48, 128, 1, 1, 4, 8, 2, 1, 0, 1, 0, 2, 3>>("32x48x128_k4_sp8_pf2_dAW"),
    make_entry<Tile<16, 96, 128, 1, 2, 2, 8, 3, 1, 1, 1, 1, 2, 2>>("16x96x128_w1x2_k2_sp8_pf3_il_cil_dW"),
    make_entry<Tile<32, 96, 128, 1, 2, 2, 8, 3, 1, 1, 2, 1, 2, 3>>("32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dAW"),
    make_entry<Tile<32, 96, 128, 1, 2, 2, 8, 3, 1, 1, 2, 1, 2, 2>>("32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dW"),
    make_entry<Tile<16, 48, 128, 1, 1, 4, 4, 2, 1, 0, 1, 0, 2, 3>>("16x48x128_k4_sp4_dAW"),
    // small grids with binary16 W over a long contraction: K split over two
    // or four workgroups
    make_entry<Tile<16, 48, 128, 1, 1, 4, 4, 2, 1, 0, 2, 0, 2, 3>>("16x48x128_k4_sp4_ks2_dAW"),
    make_entry<Tile<16, 48, 128, 1, 1, 4, 4, 2, 1, 0, 4, 0, 2, 3>>("16x48x128_k4_sp4_ks4_dAW"),
    make_entry<Tile<32, 48, 128, 1, 1, 4, 8, 2, 1, 0, 2, 0, 2, 3>>("32x48x128_k4_sp8_pf2_ks2_dAW"),
    make_entry<Tile<32, 48, 128, 1, 1, 4, 8, 2, 1, 0, 4, 0, 2, 3>>("32x48x128_k4_sp8_pf2_ks4_dAW"),
    make_entry<Tile<32, 96, 128, 1, 2, 2, 8, 3, 1, 1, 4, 1, 2, 3>>("32x96x128_w1x2_k2_sp8_pf3_il_ks4_cil_dAW"),
    // W in the compute waves' registers (fp32 W only)
    make_entry<Tile<16, 192, 128, 1, 4, 1, 4, 3, 1, 1, 2, 0, 2, 0, 4>>("16x192x128_w1x4_sp4_pf3_il_ks2_wr4"),
    make_entry<Tile<16, 96, 128, 1, 2, 2, 8, 2, 1, 1, 1, 0, 2, 0, 4>>("16x96x128_w1x2_k2_sp8_pf2_il_wr4"),
    make_entry<Tile<16, 96, 128, 1, 2, 2, 4, 3, 1, 1, 1, 0, 2, 1, 4>>("16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"),
    make_entry<Tile<16, 48, 128, 1, 1, 4, 4, 3, 1, 1, 1, 0, 2, 1, 2>>("16x48x128_k4_sp4_pf3_il_dA_wr2"),
    // the same tiles with K split over two or four workgroups (small
    // outputs over a long contraction)
    make_entry<Tile<16, 48, 128, 1, 1, 4, 4, 3, 1, 1, 2, 0, 2, 1, 2>>("16x48x128_k4_sp4_pf3_il_ks2_dA_wr2"),
    make_entry<Tile<16, 48, 128, 1, 1, 4, 4, 3, 1, 1, 4, 0, 2, 1, 2>>("16x48x128_k4_sp4_pf3_il_ks4_dA_wr2"),
    make_entry<Tile<16, 96, 128, 1, 2, 2, 4, 3, 1, 1, 2, 0, 2, 1, 4>>("16x96x128_w1x2_k2_sp4_pf3_il_ks2_dA_wr4"),
    make_entry<Tile<16, 96, 128, 1, 2, 2, 4, 3, 1, 1, 4, 0, 2, 1, 4>>("16x96x128_w1x2_k2_sp4_pf3_il_ks4_dA_wr4"),
    make_entry<Tile<16, 192, 128, 1, 4, 1, 4, 3, 1, 1, 4, 0, 2, 0, 4>>("16x192x128_w1x4_sp4_pf3_il_ks4_wr4"),
    make_entry<Tile<32, 192, 64, 1, 4, 1, 4, 3, 1, 1, 1, 0, 2, 1, 4>>("32x192x64_w1x4_sp4_pf3_il_dA_wr4"),
    make_entry<Tile<32, 384, 64, 1, 4, 1, 4, 3, 1, 1, 1, 0, 2, 1, 2>>("32x384x64_w1x4_sp4_pf3_il_dA_wr2"),
    // specialised, register staging only, two stages of loads in flight
    make_entry<Tile<128, 128, 32, 2, 2, 1, 4, 2, 1>>("128x128x32_w2x2_sp4"),
    // specialised, three stages in flight without the interleaving hint,
    // eight staging waves
    make_entry<Tile<64, 48, 64, 2, 1, 2, 8, 3, 1>>("64x48x64_w2x1_k2_sp8_pf3"),
    // K split over eight workgroups
    make_entry<Tile<128, 96, 64, 2, 2, 1, 8, 2, 1, 0, 8>>("128x96x64_w2x2_sp8_ks8"),
    // cooperative: every wave stages and computes (one, then two stages of
    // loads in flight)
    make_entry<Tile<64, 64, 64, 2, 2, 1, 0, 1, 2>>("64x64x64_w2x2"),
    make_entry<Tile<32, 48, 64, 1, 1, 4, 0, 2, 2>>("32x48x64_k4_pf2"),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

// The backward products use the configurations that the forward selection
// picks from, under the same names: fn[op == kOpTN][swiglu][accumulate].
// For matmul_t (kOpNT) the SwiGLU slot holds the fused SwiGLU backward
// (matmul_t's product dH turned into dGATE and dUP in the epilogue), which
// has no accumulating form.
template <class C>
constexpr ConfigEntry make_bwd_entry(const char *name) {
    return ConfigEntry{name, C::BM, C::BN, C::BK, C::NT, C::KS,
                       {{{gemm_fwd_kernel<C, false, false, false, kOpNT>, gemm_fwd_kernel<C, false, false, true, kOpNT>},
                         {gemm_fwd_kernel<C, false, false, false, kOpNT, kEpiSwigluBwd>, nullptr}},
                        {{gemm_fwd_kernel<C, false, false, false, kOpTN>, gemm_fwd_kernel<C, false, false, true, kOpTN>},
                         {gemm_fwd_kernel<C, true, false, false, kOpTN>, gemm_fwd_kernel<C, true, false, true, kOpTN>}}}};
}

const ConfigEntry kBwdConfigs[] = {
    make_bwd_entry<Tile<128, 128, 32, 2, 2, 1, 4, 3, 1, 1, 1, 0, 2, 1>>("128x128x32_w2x2_sp4_pf3_il_dA"),
    make_bwd_entry<Tile<128, 192, 32, 2, 2, 1, 8, 4, 1, 1>>("128x192x32_w2x2_sp8_pf4_il"),
    make_bwd_entry<Tile<64, 64, 64, 2, 2, 1, 4, 2, 1>>("64x64x64_w2x2_sp4"),
    make_bwd_entry<Tile<64, 48, 64, 2, 1, 2, 4, 3, 1, 1, 1, 0, 2, 1>>("64x48x64_w2x1_k2_sp4_pf3_il_dA"),
    make_bwd_entry<Tile<32, 48, 64, 1, 1, 4, 4, 3, 1, 0, 1, 0, 2, 3>>("32x48x64_k4_sp4_pf3_dAW"),
    make_bwd_entry<Tile<16, 96, 64, 1, 1, 4, 8, 3, 1, 1>>("16x96x64_k4_sp8_pf3_il"),
    make_bwd_entry<Tile<32, 96, 64, 1, 2, 2, 8, 3, 1, 1, 2, 1, 2, 2>>("32x96x64_w1x2_k2_sp8_pf3_il_ks2_cil_dW"),
    make_bwd_entry<Tile<16, 48, 128, 1, 1, 4, 4, 2, 1, 0, 1, 0, 2, 3>>("16x48x128_k4_sp4_dAW"),
    // long contractions on small outputs (the lm_head's dX: 512 x 16384 x 768)
    make_bwd_entry<Tile<128, 96, 64, 2, 2, 1, 8, 3, 1, 1, 8, 1, 2, 1>>("128x96x64_w2x2_sp8_pf3_il_ks8_cil_dA"),
    // transposed A whose 32 x 48 grid would leave half the CUs a second
    // tile (the attention projections' dW, 768 x 512 x 768)
    make_bwd_entry<Tile<48, 48, 64, 1, 1, 4, 4, 3, 1, 0, 1, 0, 2, 3>>("48x48x64_k4_sp4_pf3_dAW"),
    // a transposed A over a long contraction onto a small grid (the
    // 8192-token attention projections' dW): K split over two or four
    // workgroups
    make_bwd_entry<Tile<48, 48, 64, 1, 1, 4, 4, 2, 1, 0, 2, 0, 2, 3>>("48x48x64_k4_sp4_pf2_ks2_dAW"),
    make_bwd_entry<Tile<48, 48, 64, 1, 1, 4, 4, 2, 1, 0, 4, 0, 2, 3>>("48x48x64_k4_sp4_pf2_ks4_dAW"),
    // a transposed B whose grid of 128 x 64 tiles comes to two per CU
    // (the 8192-token dX of the attention projections and of gate/up)
    make_bwd_entry<Tile<128, 64, 32, 2, 2, 1, 4, 3, 1, 1, 1, 0, 2, 1>>("128x64x32_w2x2_sp4_pf3_il_dA"),
    // transposed B on the smallest grids: 128-deep slices two at a time
    make_bwd_entry<Tile<32, 48, 128, 1, 1, 4, 8, 2, 1, 0, 1, 0, 2, 3>>("32x48x128_k4_sp8_pf2_dAW"),
    // a transposed B over a long contraction onto a small grid: K split
    // over two, four or eight workgroups
    make_bwd_entry<Tile<16, 48, 128, 1, 1, 4, 4, 2, 1, 0, 2, 0, 2, 3>>("16x48x128_k4_sp4_ks2_dAW"),
    make_bwd_entry<Tile<16, 48, 128, 1, 1, 4, 4, 2, 1, 0, 4, 0, 2, 3>>("16x48x128_k4_sp4_ks4_dAW"),
    make_bwd_entry<Tile<16, 48, 128, 1, 1, 4, 4, 2, 1, 0, 8, 0, 2, 3>>("16x48x128_k4_sp4_ks8_dAW"),
    make_bwd_entry<Tile<32, 48, 128, 1, 1, 4, 8, 2, 1, 0, 2, 0, 2, 3>>("32x48x128_k4_sp8_pf2_ks2_dAW"),
    make_bwd_entry<Tile<32, 48, 128, 1, 1, 4, 8, 2, 1, 0, 4, 0, 2, 3>>("32x48x128_k4_sp8_pf2_ks4_dAW"),
    make_bwd_entry<Tile<32, 48, 128, 1, 1, 4, 8, 2, 1, 0, 8, 0, 2, 3>>("32x48x128_k4_sp8_pf2_ks8_dAW"),
    // weight gradients over a short contraction: dY (B in its natural
    // layout) straight into the compute waves' registers
    make_bwd_entry<Tile<32, 96, 128, 1, 2, 2, 4, 3, 1, 1, 1, 0, 2, 1, 4>>("32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"),
};
constexpr int kNumBwdConfigs = sizeof(kBwdConfigs) / sizeof(kBwdConfigs[0]);

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The forward choice splits K over workgroups only for outputs of at most
// this many elements: the range where it was measured to win (larger outputs
// fill the CUs without it).  The backward choice has one exception of its
// own, the one-round 48 x 48 grid over a long contraction.
constexpr int64_t kSplitMaxElems = (int64_t)1 << 19;

// Workspace layout: a fixed block of kCounterBytes holding one arrival
// counter per output tile (so a call never finds another call's partial
// tiles where its counters are: only the counters are left zero after a
// call), then KS partial slots of M x N floats.
constexpr int64_t kCounterBytes = 64 << 10;
constexpr int64_t kMaxSplitTiles = kCounterBytes / 4;
// Size of the library-held workspace of gemm_fwd_swiglu_noalloc (below).
constexpr int64_t kScratchBytes = kCounterBytes + (4 << 20);

// Bytes a split-K configuration needs for an M x N output; zero for a
// configuration without split-K, -1 for one with more output tiles than the
// counter block holds.
int64_t split_workspace_bytes(const ConfigEntry &e, int64_t M, int64_t N) {
    if (e.ks <= 1) return 0;
    const int64_t tiles = ceil_div(M, e.bm) * ceil_div(N, e.bn);
    if (tiles > kMaxSplitTiles) return -1;
    return kCounterBytes + (int64_t)e.ks * M * N * 4;
}

int table_index(const ConfigEntry *table, int count, const char *name) {
    for (int i = 0; i < count; ++i) {
        const char *a = table[i].name, *b = name;
        while (*a && *a == *b) ++a, ++b;
        if (*a == 0 && *b == 0) return i;
    }
    return -1;
}
int config_index(const char *name) { return table_index(kConfigs, kNumConfigs, name); }

bool same_name(const char *a, const char *b) {
    while (*a && *a == *b) ++a, ++b;
    return *a == 0 && *b == 0;
}

// Choosing among tiles and K splits by estimated time (small outputs over a
// long contraction).  The estimate: the rounds of workgroups over the 256
// CUs, times each workgroup's contraction, times its area in units of
// 16 x 48 outputs (plus, with SwiGLU, half a unit per 16 rows for the
// combine, done once per tile), and 1.2 times that for 16 x 48 tiles alone
// on their CUs (24 MFMAs per wave between barriers, with no second
// workgroup to fill the waits).  A split keeps 512 or more of the
// contraction per workgroup (1024 or more where the split grid exceeds two
// workgroups per CU), at most max_wgs workgroups and 2^20 partial elements.
// Ties keep `base` (a negative base_cost: the base never stays); among
// candidates of equal estimate the first listed wins.
struct SplitCand { int bm, bn, ks; const char *name; };

double split_estimate(int64_t M, int64_t K, int64_t N, bool swiglu, int bm, int bn, int ks) {
    const int64_t cus = 256;
    const int64_t wgs = ceil_div(M, bm) * ceil_div(N, bn) * ks;
    return (double)ceil_div(wgs, cus) * (double)ceil_div(K, ks) * (bm * bn / 768.0 + (swiglu ? bm / 32.0 : 0.0)) *
           (bm == 16 && bn == 48 && wgs <= cus ? 1.2 : 1.0);
}

const char *pick_by_estimate(int64_t M, int64_t K, int64_t N, bool swiglu, bool splits, int64_t max_wgs,
                             const SplitCand *cands, int count, const char *base, double base_cost) {
    const int64_t cus = 256;
    const char *best = base;
    double best_cost = base_cost < 0 ? 1e300 : base_cost;
    for (int i = 0; i < count; ++i) {
        const SplitCand &c = cands[i];
        const int64_t wgs = ceil_div(M, c.bm) * ceil_div(N, c.bn) * c.ks;
        if (c.ks > 1 && (!splits || K / c.ks < (wgs > 2 * cus ? 1024 : 512) || wgs > max_wgs ||
                         c.ks * M * N > ((int64_t)1 << 20)))
            continue;
        const double t = split_estimate(M, K, N, swiglu, c.bm, c.bn, c.ks);
        if (t < best_cost) best = c.name, best_cost = t;
    }
    return best;
}

// Tile choice from the output grid, measured on MI355X: the largest tile
// that still gives every CU work for the whole kernel, then narrower tiles
// with the K range split over waves for small grids.  With SwiGLU, a
// 64 x 384 tile re-stages (and recombines) each block of A rows half as
// often as 128 x 192 at the same MFMA work per wave: 297 against 310 us at
// 8192 x 3072 x 768 with f16 W, 298 against 309 with fp32 W; with fp32 W,
// 32 x 384 tiles with W in registers do better still (278 against 300 us
// there, 280 against 311 and 352 for 128 x 128 at 8192 x 1536 x 1536, 1105
// against 1220 and 1386 at 16384 x 3072 x 1536), and 32 x 192 ones where N
// is far from a multiple of 384 (8191 x 3072 x 772: 361 against 409, and
// 586 for 64 x 384; 8192 x 4096 x 2048: 1067 against 1090, and 1205 for
// 128 x 128).  Other grids
// too small for 128 x 128 take 128 x 64 tiles while those come to two per
// CU: 512 x 768 x 8192 in 51.6 us against 56.8 for 64 x 64; 8192 x 768 x 768
// in 77 against 86 us (f16 W) and 75 against 79 (fp32 W with R) for
// 128 x 192; 8192 x 3072 x 768 with f16 W in 279 against 295; never slower
// than 128 x 192 on the shapes measured.  And 64 x 64 tiles
// rather than 64 x 48 where the 64 x 64 grid is one whole round of the CUs
// and the 64 x 48 one is not (512 x 768 x 2048: 17.8 against 21.8 us).
// Where 128 x 48 tiles fill the CUs and larger ones do not, forward products
// take them rather than 64 x 48 (two per CU): 21.7 against 22.0 us at
// 512 x 768 x 3072 with f16 W, 32.9 against 36.2 at 1024 x 768 x 1536 and
// 40.6 against 44.3 at 2048 x 1024 x 768 with SwiGLU, level (within 0.5%)
// at 2048 x 768 x 768 and 512 x 1024 x 3072.
// With f16 W (and in the backward rule), the smallest grids stage 128-deep
// slices of K two at a time with eight staging waves (measured with fp32 W
// before the tiles below existed: at 512 x 768 x 768, one 32 x 48 tile per
// CU, 7.6 against 9.3 us with 64-deep slices three at a time and four
// staging waves; 16.1 against 17.5 us at 512 x 1536 x 768 with SwiGLU; one
// shape measured the other way: 512 x 1024 x 1024 with f16 W, 18.7 against
// 17.2 us), and a long K splits over two workgroups when the caller provides
// a workspace (`split`), with 128-deep slices, or without one takes 16 x 96
// tiles over the whole K (measured with fp32 W: 26.6 against 39.2 us for
// 64-deep slices split over four waves at 512 x 3072 x 768 with SwiGLU).
// Grids below those of the larger tiles, with fp32 W (forward products
// only), take tiles that keep W in the compute waves' registers, so that the
// LDS holds A alone; W16 tiles of that kind do not exist.  32 x 192 tiles
// where their grid fills whole rounds of the 256 CUs (2048 x 768 x 768: 20.9
// against 21.8 us for 128 x 48; 1024 x 768 x 1536 with SwiGLU: 23.7 against
// 32.2).  With SwiGLU and a long K and a workspace: 16 x 192 tiles with K
// split in two, which combine each element of A four times instead of eight
// (512 x 3072 x 768: 24.0 against 26.0 us for 32 x 96 tiles with W staged
// through LDS).  Otherwise 16 x 96 tiles, or 16 x 48 where their grid fills
// whole rounds better (for SwiGLU, which they combine twice as often, only
// when the 16 x 96 grid is below one round): 512 x 1024 x 1024 in 12.7
// against 14.6 us for 16 x 96 and 16.6 for 32 x 48 with W in LDS,
// 128 x 768 x 768 in 4.5 against 5.8, 1000 x 768 x 772 in 14.9 against 17.3;
// with SwiGLU 128 x 3072 x 768 in 17.2 against 24.3, but 768 x 768 x 2048 in
// 32.0 on 16 x 96 against 33.2 (and 59.8 for 128 x 48).  With SwiGLU the
// 16 x 96 tiles use eight staging waves up to one round (24.9 against 26.6 us
// at 512 x 3072 x 768 without a workspace) and four beyond, where two
// workgroups then share a CU (2000 x 1000 x 780: 40.6 against 44.8).  A
// plain A at 512 x 3072 x 768 is not split over workgroups (20.8 us for
// 16 x 96 against 21.9 for the fastest split); smaller outputs over long
// contractions are (pick_by_estimate, below).
// `forward` false: the rule as the backward products measured it, without
// the 128 x 64 and 128 x 48 tiles, the whole-round 64 x 64 choice, the
// 128-deep slices and W in registers; every name it gives is in the
// backward table.
const char *select_rule(int64_t M, int64_t K, int64_t N, int swiglu, int w16, bool split, bool forward) {
    const int64_t cus = 256;
    // Products with few columns (a narrow W, or the input gradient of a
    // narrow layer): no tile more than twice as wide as the columns it
    // covers, since most of its MFMA work would be padding (8192 x 768 x 48
    // with fp32 W: 7.0 against 20.1 us on 32 x 192; 32768 x 768 x 64: 27.7
    // on 64 x 64 against 72.8 on 128 x 192; matmul_t onto 32768 x 64: 30.6
    // on 64 x 64 against 78.0 on 128 x 192).
    auto cols = [&](int bn) { return N * 2 > ceil_div(N, bn) * bn; };
    const bool wide_swiglu = swiglu && ceil_div(M, 64) * ceil_div(N, 384) >= cus;
    // SwiGLU with fp32 W on a large grid (ahead of 128 x 128, which combines
    // each element of A once per 128 columns): 32 x 384 tiles with W in
    // registers, or 32 x 192 where 384-wide tiles would leave more than a
    // tenth of their columns past N
    if (wide_swiglu && forward && !w16 && cols(192))
        return ceil_div(N, 384) * 384 * 10 <= N * 11 ? "32x384x64_w1x4_sp4_pf3_il_dA_wr2"
                                                      : "32x192x64_w1x4_sp4_pf3_il_dA_wr4";
    // Forward products with few rows (decoding a few tokens against a wide
    // W): no 128-row tiles for 64 rows or fewer, no 64-row tiles for 32 or
    // fewer, however many columns, as most of such a tile's MFMA work would
    // be padding; with fp32 W, whose 16-row tiles hold W in registers, no
    // 64-row tiles over more than one round for 48 or fewer either (the one
    // whole round of 64 x 64 tiles below stays).  16 x 768 x 50304 with
    // binary16 W: 23.1 against 95.2 us on 128 x 64; 16 x 768 x 16384: 9.4
    // against 16.4 on 64 x 64; 48 x 768 x 50304 with fp32 W: 37.8 against
    // 95.2 (128 x 64) and 50.9 (64 x 64); 64 x 4096 x 50304 with binary16 W:
    // 259 against 489 us on 128 x 64.
    const bool rows128 = !forward || M > 64, rows64 = !forward || M > (w16 ? 32 : 48);
    const bool rows64_round = !forward || M > 32;
    // forward products: 128 x 128 only where its grid fills 70% or more of
    // the rounds of two workgroups per CU it takes (576 tiles, 3072 x K x
    // 3072, take 1.125 rounds: 138 against 118 us on 128 x 64 with binary16
    // W at 3072 x 768 x 3072, 109 on 32 x 192 with fp32 W)
    const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128);
    const bool fill128 = !forward || t128 * 10 >= ceil_div(t128, 2 * cus) * 2 * cus * 7;
    if (rows128 && cols(128) && fill128 && t128 >= 2 * cus) return "128x128x32_w2x2_sp4_pf3_il_dA";
    if (rows64 && cols(384) && wide_swiglu) return "64x384x32_w1x4_sp8_pf4_il";
    // forward products: 128 x 64 wherever that gives two tiles per CU, which
    // covers every grid 128 x 192 would fill; the backward rule keeps 128 x 192
    const int64_t t128x64 = ceil_div(M, 128) * ceil_div(N, 64);
    if (rows128 && cols(64) && forward && t128x64 >= 2 * cus) {
        if (t128x64 * 10 >= ceil_div(t128x64, 2 * cus) * 2 * cus * 7) return "128x64x32_w2x2_sp4_pf3_il_dA";
        // a 128 x 64 grid filling under 70% of its rounds of two per CU (576
        // tiles at 3072 x 768 x 1536 took 72 us): fp32 W in registers on
        // 32 x 192 tiles where their grid fills whole rounds (55), f16 W
        // without SwiGLU on 128 x 48 tiles where theirs fills whole rounds of
        // three per CU (58); otherwise on to the 64 x 64 tiles (68, and 83
        // against 105 with SwiGLU), which without SwiGLU lost where the grid
        // fills 60% or more (648 tiles at 2304 x 768 x 2304: 79 against 72)
        const int64_t t32w = ceil_div(M, 32) * ceil_div(N, 192), t128x48 = ceil_div(M, 128) * ceil_div(N, 48);
        if (!w16 && cols(192) && t32w * 10 >= ceil_div(t32w, cus) * cus * 9) return "32x192x64_w1x4_sp4_pf3_il_dA_wr4";
        if (w16 && !swiglu && t128x48 * 10 >= ceil_div(t128x48, 3 * cus) * 3 * cus * 9)
            return "128x48x32_w2x1_k2_sp4_pf3_il_dA";
        if (!swiglu && t128x64 * 10 >= ceil_div(t128x64, 2 * cus) * 2 * cus * 6) return "128x64x32_w2x2_sp4_pf3_il_dA";
        if (rows64) return "64x64x64_w2x2_sp4_dAW";
    }
    if (rows128 && cols(192) && ceil_div(M, 128) * ceil_div(N, 192) >= cus) return "128x192x32_w2x2_sp8_pf4_il";
    const int64_t t64 = ceil_div(M, 64) * ceil_div(N, 64), t48 = ceil_div(M, 64) * ceil_div(N, 48);
    if (rows64 && cols(64) && t64 >= 2 * cus) {
        // a forward 64 x 64 grid filling under 70% of its rounds of two per
        // CU (576 tiles at 1536 x 768 x 1536: 39.5 us with fp32 W, 42.6 with
        // f16 W, 49.1 with SwiGLU): 64 x 48 tiles without SwiGLU where their
        // grid fills whole rounds of three per CU (33.5, 32.7), else fp32 W
        // in registers on 32 x 192 tiles (37.0, 41.0 with SwiGLU) and f16 W
        // without SwiGLU on 128 x 48 tiles where their grid fills three
        // quarters of its rounds of two per CU (38.9 at 1536 x 768 x 1536,
        // 39.0 against 42.2 at 2304 x 768 x 1152; 544 tiles at 448 x 768 x
        // 6528 took 57.2 against 42.6); f16 W with SwiGLU stays
        const int64_t t64x48 = ceil_div(M, 64) * ceil_div(N, 48);
        if (forward && t64 * 10 < ceil_div(t64, 2 * cus) * 2 * cus * 7) {
            if (!swiglu && t64x48 * 10 >= ceil_div(t64x48, 3 * cus) * 3 * cus * 9) return "64x48x64_w2x1_k2_sp4_pf3_il_dA";
            if (!w16 && cols(192)) return "32x192x64_w1x4_sp4_pf3_il_dA_wr4";
            const int64_t t128x48 = ceil_div(M, 128) * ceil_div(N, 48);
            if (w16 && !swiglu && rows128 && t128x48 * 4 >= ceil_div(t128x48, 2 * cus) * 2 * cus * 3)
                return "128x48x32_w2x1_k2_sp4_pf3_il_dA";
        }
        return "64x64x64_w2x2_sp4_dAW";
    }
    if (rows64_round && cols(64) && forward && t48 >= cus && t48 < 2 * cus && t64 * 10 >= cus * 9 && t64 <= cus) {
        // over a contraction of 2048 or more with a workspace, K split in
        // two: two workgroups per CU instead of one (1024 x 4096 x 1024:
        // 67.2 against 71.8 us with fp32 W, 70.9 against 77.3 with binary16
        // W; 1024 x 8192 x 1024: 129.6 against 141.0; at a contraction of
        // 1024 the split lost, 21.3 against 20.2); with SwiGLU only while
        // the partial tiles fit the allocation-free entry point's scratch
        if (split && K >= 2048 && (!swiglu || 2 * M * N <= ((int64_t)1 << 20))) return "64x64x64_w2x2_sp4_ks2_dAW";
        return "64x64x64_w2x2_sp4_dAW";
    }
    // the fraction of whole rounds of the CUs a grid of t tiles keeps busy
    auto fill = [&](int64_t t) { return (double)t / (double)(ceil_div(t, cus) * cus); };
    if (forward && !w16) {
        // every smaller grid with fp32 W: tiles with W in registers; 32 x 192
        // where that grid fills whole rounds of the CUs (nine tenths or more)
        const int64_t t32w = ceil_div(M, 32) * ceil_div(N, 192);
        if (cols(192) && t32w >= cus && fill(t32w) >= 0.9) return "32x192x64_w1x4_sp4_pf3_il_dA_wr4";
        if (swiglu && cols(192) && K >= 2048 && split && M * N <= kSplitMaxElems &&
            ceil_div(M, 16) * ceil_div(N, 192) * 2 >= cus)
            return "16x192x128_w1x4_sp4_pf3_il_ks2_wr4";
        // 16 x 48 where its grid fills whole rounds better, counting only
        // the columns each tile covers (with SwiGLU, which it then combines
        // more often, only below one round of 16 x 96)
        const int64_t s96 = ceil_div(M, 16) * ceil_div(N, 96), s48 = ceil_div(M, 16) * ceil_div(N, 48);
        const double u96 = (double)N / (double)(ceil_div(N, 96) * 96), u48 = (double)N / (double)(ceil_div(N, 48) * 48);
        const bool more48 = ceil_div(N, 48) > ceil_div(N, 96);
        const char *base = fill(s96) * u96 < fill(s48) * u48 && (!swiglu || !more48 || s96 < cus)
                               ? "16x48x128_k4_sp4_pf3_il_dA_wr2"
                           // SwiGLU on one round at most: eight staging
                           // waves; otherwise four, which lets two
                           // workgroups share a CU
                           : swiglu && s96 <= cus ? "16x96x128_w1x2_k2_sp8_pf2_il_wr4"
                                                  : "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4";
        // Over a long contraction with a workspace: the 16-row tile (48, 96
        // or 192 wide) and K split (none, two or four workgroups) of least
        // estimated time (pick_by_estimate).  Not below 3072 for grids of
        // more than half a round (splits there lost up to 18%), nor below
        // 8192 for the eight-staging-wave SwiGLU tile (0.81 to 1.14 times as
        // fast).  Against the choice above, over 16 to 768 rows,
        // contractions of 2048 to 16384 and 512 to 2048 columns: 1.6 times
        // as fast on the geometric mean, up to 3.4 (64 x 3072 x 768 with
        // SwiGLU 17.2 -> 8.3 us, 128 x 8192 x 768 37 -> 18 us).
        const bool base48 = same_name(base, "16x48x128_k4_sp4_pf3_il_dA_wr2");
        const bool sp8 = same_name(base, "16x96x128_w1x2_k2_sp8_pf2_il_wr4");
        if (!split || K < (sp8 ? 8192 : 2048) || (K < 3072 && (base48 ? s48 : s96) > cus / 2)) return base;
        static const SplitCand cands[] = {
            {16, 48, 1, "16x48x128_k4_sp4_pf3_il_dA_wr2"},         {16, 96, 1, "16x96x128_w1x2_k2_sp4_pf3_il_dA_wr4"},
            {16, 48, 2, "16x48x128_k4_sp4_pf3_il_ks2_dA_wr2"},     {16, 96, 2, "16x96x128_w1x2_k2_sp4_pf3_il_ks2_dA_wr4"},
            {16, 192, 2, "16x192x128_w1x4_sp4_pf3_il_ks2_wr4"},    {16, 48, 4, "16x48x128_k4_sp4_pf3_il_ks4_dA_wr2"},
            {16, 96, 4, "16x96x128_w1x2_k2_sp4_pf3_il_ks4_dA_wr4"}, {16, 192, 4, "16x192x128_w1x4_sp4_pf3_il_ks4_wr4"}};
        return pick_by_estimate(M, K, N, swiglu, true, INT64_MAX, cands, sizeof(cands) / sizeof(cands[0]), base,
                                split_estimate(M, K, N, swiglu, 16, base48 ? 48 : 96, 1));
    }
    // forward products: 128 x 48 where that grid fills the CUs, which stages
    // (and widens, or combines) each block of W (or A) half as often
    if (rows128 && forward && ceil_div(M, 128) * ceil_div(N, 48) >= cus) return "128x48x32_w2x1_k2_sp4_pf3_il_dA";
    if (rows64 && t48 >= cus) return "64x48x64_w2x1_k2_sp4_pf3_il_dA";
    const char *small = nullptr;
    if (M <= 128) small = "16x48x128_k4_sp4_dAW";
    else if (K >= 2048) {
        // long K on a small grid: split K in two when there is a workspace
        // (for outputs up to 2^19 elements, the range measured)
        if (split && M * N <= kSplitMaxElems && ceil_div(M, 32) * ceil_div(N, 96) * 2 >= cus) {
            if (!forward) return "32x96x64_w1x2_k2_sp8_pf3_il_ks2_cil_dW";
            small = swiglu ? "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dW" : "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dAW";
        } else {
            small = forward ? "16x96x128_w1x2_k2_sp8_pf3_il_cil_dW" : "16x96x64_k4_sp8_pf3_il";
        }
    } else {
        small = forward ? "32x48x128_k4_sp8_pf2_dAW" : "32x48x64_k4_sp4_pf3_dAW";
    }
    if (!forward || !split || K < 2048) return small;
    // The forward products with binary16 W over a long contraction with a
    // workspace: the tile and K split of least estimated time
    // (pick_by_estimate; not below 3072 for grids of more than half a
    // round), the 32-row tiles listed first so that equal estimates take
    // fewer and larger workgroups.  SwiGLU takes the 32 x 96 two-way split
    // in its W-only DMA form, as above.  64 x 3072 x 768 with SwiGLU:
    // 21.5 -> 9.7 us; 128 x 8192 x 768: 42.9 -> 20.2 us; 32 x 4096 x 1024:
    // 22.4 -> 9.8 us.
    const SplitCand cands[] = {
        {32, 48, 1, "32x48x128_k4_sp8_pf2_dAW"},     {32, 48, 2, "32x48x128_k4_sp8_pf2_ks2_dAW"},
        {32, 48, 4, "32x48x128_k4_sp8_pf2_ks4_dAW"}, {16, 48, 1, "16x48x128_k4_sp4_dAW"},
        {16, 48, 2, "16x48x128_k4_sp4_ks2_dAW"},     {16, 48, 4, "16x48x128_k4_sp4_ks4_dAW"},
        {16, 96, 1, "16x96x128_w1x2_k2_sp8_pf3_il_cil_dW"},
        {32, 96, 2, swiglu ? "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dW" : "32x96x128_w1x2_k2_sp8_pf3_il_ks2_cil_dAW"},
        {32, 96, 4, "32x96x128_w1x2_k2_sp8_pf3_il_ks4_cil_dAW"}};
    const int count = sizeof(cands) / sizeof(cands[0]);
    const SplitCand *base = nullptr;
    for (const SplitCand &c : cands)
        if (same_name(c.name, small)) base = &c;
    if (base == nullptr || (K < 3072 && ceil_div(M, base->bm) * ceil_div(N, base->bn) > cus / 2)) return small;
    return pick_by_estimate(M, K, N, swiglu, true, INT64_MAX, cands, count, small,
                            split_estimate(M, K, N, swiglu, base->bm, base->bn, base->ks));
}

// The forward choice: an index into kConfigs (-1 if the rule names a tile
// the table lacks, which would be a build error in spirit).
int select_config(int64_t M, int64_t K, int64_t N, int swiglu, int w16, bool split) {
    return config_index(select_rule(M, K, N, swiglu, w16, split, true));
}

// Tile choice for the backward products, by their kernel dimensions (output
// rows, contraction, output columns): the shared rule (select_rule with
// `forward` false), with these exceptions measured on the seq-512 model's
// backward shapes and their 8192-token batch.  A transposed A is read with
// four LDS reads per fragment, so with a short contraction the 64 x 64
// tiles lose to 32 x 48 tiles with the K range split over four waves (about
// 20% at 768 x 512 x 3072 and 3072 x 512 x 768).  With a transposed B and a
// contraction of a few thousand, 16 x 48 tiles with BK = 128 beat the
// two-workgroup split-K (6% at 512 x 3072 x 768).  With a contraction of
// 8192 or more, 128 x 96 tiles with the K range split eight ways re-read the
// transposed B a quarter as often as 32 x 96 tiles and win by 12% (the
// lm_head's dX, 512 x 16384 x 768).  Where those 32 x 48 tiles of a
// transposed A come to between one and two per CU while 48 x 48 tiles come
// to at most one, the 48 x 48 tiles finish in one round: 9.7 against 10.8 us
// at 768 x 512 x 768.  Over a contraction of 1024 or more, grids of up to
// two rounds of 48 x 48 tiles take those tiles with K split over two or
// four workgroups (below).  Otherwise weight gradients whose
// 32 x 96 grid fills whole rounds of the CUs (three quarters of each round
// or more) take 32 x 96 tiles that load dY straight into the compute waves'
// registers (LDS then holds the transposed A alone), whatever the
// contraction: 23.2 against 24.9 us at 768 x 512 x 3072 (24.1 against 25.7
// accumulating), 26.4 against 27.7 at 3072 x 512 x 768 with SwiGLU, 283
// against 311 (48 x 48) at 768 x 8192 x 3072, 314 against 347 (96 x 96, which
// combines G and U half as often as 48-wide tiles) at 3072 x 8192 x 768 with
// SwiGLU, 558 against 608 at 768 x 16384 x 3072; at 1024 x 2048 x 1024, whose
// 32 x 96 grid leaves most of a second round idle, 48.8 against 43.0.  A
// transposed B takes 128 x 64 tiles where they come to two per CU and
// 128 x 128 tiles do not: 74 against 80 us at 8192 x 768 x 768 and 282
// against over 300 at 8192 x 3072 x 768.  The split-K tiles need the
// caller's workspace (`split`).
int select_bwd_rule(int op, int64_t M, int64_t K, int64_t N, int swiglu, bool split) {
    static const char *const fwd_mid = "64x64x64_w2x2_sp4_dAW", *const mid = "64x64x64_w2x2_sp4";
    static const char *const deep = "16x96x64_k4_sp8_pf3_il";
    static const char *const deep_split = "32x96x64_w1x2_k2_sp8_pf3_il_ks2_cil_dW";
    static const char *const small = "32x48x64_k4_sp4_pf3_dAW";
    auto bwd = [](const char *name) { return table_index(kBwdConfigs, kNumBwdConfigs, name); };
    const int64_t cus = 256;
    // the shared rule without its SwiGLU and forward-only tiles, which the
    // backward table does not hold
    const char *f = select_rule(M, K, N, 0, 0, split, false);
    if (op == kOpNT && ceil_div(M, 128) * ceil_div(N, 64) >= 2 * cus && ceil_div(M, 128) * ceil_div(N, 128) < 2 * cus)
        return bwd("128x64x32_w2x2_sp4_pf3_il_dA");
    // without split-K the rule's long-K choice is the deep tile
    const bool long_k_grid = same_name(f, deep_split) || (!split && same_name(f, deep));
    if (op == kOpNT && long_k_grid && K <= 4096) return bwd("16x48x128_k4_sp4_dAW");
    if (split && op == kOpNT && same_name(f, deep_split) && K >= 8192 && M * N <= kSplitMaxElems &&
        ceil_div(M, 128) * ceil_div(N, 96) * 8 >= 128)
        return bwd("128x96x64_w2x2_sp8_pf3_il_ks8_cil_dA");
    // A transposed A over a contraction of 1024 or more onto at most two
    // rounds of 48 x 48 tiles takes those tiles, with K split over as many
    // workgroups (two or four) as keep 512 or more of the contraction each
    // and the grid within one workgroup per CU below 2048 of contraction,
    // two from there; a two-way split may also take up to four per CU where
    // each keeps 4096 or more (three fit a CU at once, so four-way splits
    // of grids already at two per CU lose: 768 x 16384 x 768, 185 against
    // 154 us).  Measured over 1024 to 16384 tokens onto 512 x 512 to
    // 768 x 1536 outputs: within 3% of the best tile tried everywhere, and
    // up to 2.2x faster than the shared rule's tiles (512 x 8192 x 512: 43
    // against 95 us; 1024 x 8192 x 1024: 148 against 209 us).
    if (op == kOpTN && K >= 1024) {
        const int64_t t48 = ceil_div(M, 48) * ceil_div(N, 48);
        if (t48 <= 2 * cus) {
            int ks = 1;
            for (const int s : {2, 4}) {
                const int64_t per = K / s, wgs = t48 * s;
                if (split && per >= 512 &&
                    (wgs <= (K >= 2048 ? 2 : 1) * cus || (s == 2 && per >= 4096 && wgs <= 4 * cus)))
                    ks = s;
            }
            return bwd(ks == 4 ? "48x48x64_k4_sp4_pf2_ks4_dAW"
                               : ks == 2 ? "48x48x64_k4_sp4_pf2_ks2_dAW" : "48x48x64_k4_sp4_pf3_dAW");
        }
    }
    // a transposed A takes 32 x 48 tiles where the rule takes 64 x 64
    // (whose backward form stages with registers)
    // a transposed A where the rule's 128 x 128 grid spans more than one
    // round of two workgroups per CU but fills under 70% of the rounds it
    // takes: the 32 x 96 tiles with dY in registers, where their own grid
    // fills three quarters of its rounds or more (3072 x 1024 x 3072: 151.7
    // against 188.5 us; 3072 x 2048 x 3072: 291 against 372; where
    // 128 x 128 fills its rounds, as at 4096 x 1024 x 4096, it stays)
    if (op == kOpTN && same_name(f, "128x128x32_w2x2_sp4_pf3_il_dA")) {
        const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128), t96 = ceil_div(M, 32) * ceil_div(N, 96);
        const double fill128 = (double)t128 / (double)(ceil_div(t128, 2 * cus) * 2 * cus);
        const double fill96 = (double)t96 / (double)(ceil_div(t96, cus) * cus);
        if (t128 > 2 * cus && fill128 < 0.7 && fill96 >= 0.75) return bwd("32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4");
    }
    // the rule's 128 x 192 grid past one round of one workgroup per CU: the
    // 32 x 96 tiles where their grid fills three quarters of its rounds
    // (4096 x 4096 x 3072, two whole rounds: 745 against 782 us; 3072 x 1024
    // x 3072, 384 tiles: 152.7 against 202.2; 4608 x 4096 x 1792, 360 tiles:
    // 1.5x), else 64 x 64 tiles where it fills under 70% of its rounds
    // (2304 x 1024 x 3072: 127.3 against 200.7); one whole round stays
    // (1024 x 512 x 6144 with SwiGLU: 58.6 against 64.2 on 32 x 96)
    if (op == kOpTN && same_name(f, "128x192x32_w2x2_sp8_pf4_il")) {
        const int64_t t192 = ceil_div(M, 128) * ceil_div(N, 192), t96 = ceil_div(M, 32) * ceil_div(N, 96);
        const double fill192 = (double)t192 / (double)(ceil_div(t192, cus) * cus);
        const double fill96 = (double)t96 / (double)(ceil_div(t96, cus) * cus);
        if (t192 > cus && fill96 >= 0.75) return bwd("32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4");
        if (t192 > cus && fill192 < 0.7) return bwd("64x64x64_w2x2_sp4");
    }
    // a transposed B where the rule's 128 x 128 grid spans more than one
    // round of two workgroups per CU but fills under 70% of the rounds it
    // takes: 128 x 64 tiles (dX onto 3072 x 3072, contraction 768: 118.5
    // against 142 us; contraction 3072: 456 against 548)
    if (op == kOpNT && same_name(f, "128x128x32_w2x2_sp4_pf3_il_dA")) {
        const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128);
        if (t128 > 2 * cus && t128 * 10 < ceil_div(t128, 2 * cus) * 2 * cus * 7)
            return bwd("128x64x32_w2x2_sp4_pf3_il_dA");
    }
    const char *r = same_name(f, fwd_mid) ? (op == kOpTN ? small : mid) : f;
    // a transposed B where the rule takes 64 x 64: 64 x 48 tiles whenever
    // 48-wide tiles cover the columns at least as fully (dX onto 96 columns
    // over 16384 tokens, contraction 3072: 77.6 against 102.4 us; onto 192
    // and 384 columns 4-5% faster; onto 256, where 48-wide tiles leave a
    // ninth of their columns past N, 64 x 64 stays, 7% faster)
    if (op == kOpNT && same_name(r, mid) && N * 64 * ceil_div(N, 64) >= N * 48 * ceil_div(N, 48))
        return bwd("64x48x64_w2x1_k2_sp4_pf3_il_dA");
    auto fill = [&](int64_t t) { return (double)t / (double)(ceil_div(t, cus) * cus); };
    const bool tn_small = op == kOpTN && (same_name(r, small) || same_name(f, deep));
    // a transposed B on the smallest grids: 128-deep slices, eight staging
    // waves (qkvo dX, 512 x 768 x 768: 8.3 against 9.0 us for 64-deep ones)
    if (op == kOpNT && same_name(r, small)) return bwd("32x48x128_k4_sp8_pf2_dAW");
    if (tn_small) {
        const int64_t t32 = ceil_div(M, 32) * ceil_div(N, 48), t48 = ceil_div(M, 48) * ceil_div(N, 48);
        if (t32 > cus && t32 < 2 * cus && t48 <= cus) return bwd("48x48x64_k4_sp4_pf3_dAW");
        // dY into registers where the 32 x 96 grid fills whole rounds
        const int64_t t96 = ceil_div(M, 32) * ceil_div(N, 96);
        if (t96 >= cus && fill(t96) >= 0.75) return bwd("32x96x128_w1x2_k2_sp4_pf3_il_dA_wr4");
    }
    return bwd(r);
}

// A transposed B (matmul_t) over a contraction of 2048 or more, where the
// rule above lands on one of its small-grid tiles: the 32 x 48 or 16 x 48
// tile and K split (none, or with a workspace two, four or eight
// workgroups) of least estimated time, as for the forward products (the
// rounds of workgroups over the CUs, times each one's contraction, times its
// area in 16 x 48 units, 1.2 times that for 16 x 48 tiles alone on their
// CUs; each split keeps 512 or more of the contraction, 1024 or more past two
// workgroups per CU, the grid stays within six per CU and the partial tiles
// within 2^20 elements; ties keep the rule's tile).  Splits only from 8192
// where the 16 x 48 grid exceeds half a round: below that they measured up
// to 15% slower.  The rule's 16 x 96 x 64 tile never stays: for a transposed
// B it measured 2 to 2.4 times as slow as 16 x 48 tiles everywhere.  dX over
// 64 tokens of the lm_head (64 x 16384 x 768): 64.5 -> 20.1 us; over 256
// tokens, with or without a workspace: 159 -> 60 or 66 us.
int select_bwd_config(int op, int64_t M, int64_t K, int64_t N, int swiglu, bool split) {
    const int r = select_bwd_rule(op, M, K, N, swiglu, split);
    // a transposed B whose 128 x 64 or 64 x 64 grid spans more than one round
    // of two workgroups per CU but fills under 60% of the rounds it takes:
    // 64 x 48 tiles (512 x 1536 x 4352: 59.3 against 80.7 us on 64 x 64;
    // 1024 x 1536 x 4352: 114.6 against 138.9 on 128 x 64; 2048 x 3072 x
    // 2304: 223.2 against 274.4)
    if (op == kOpNT && r >= 0 &&
        (same_name(kBwdConfigs[r].name, "128x64x32_w2x2_sp4_pf3_il_dA") ||
         same_name(kBwdConfigs[r].name, "64x64x64_w2x2_sp4"))) {
        const int64_t t = ceil_div(M, kBwdConfigs[r].bm) * ceil_div(N, kBwdConfigs[r].bn);
        if (t > 512 && t * 10 < ceil_div(t, 512) * 512 * 6)
            return table_index(kBwdConfigs, kNumBwdConfigs, "64x48x64_w2x1_k2_sp4_pf3_il_dA");
    }
    if (op != kOpNT || K < 2048 || r < 0) return r;
    const ConfigEntry &e = kBwdConfigs[r];
    const bool deep = same_name(e.name, "16x96x64_k4_sp8_pf3_il");
    static const char *const small_tiles[] = {"16x48x128_k4_sp4_dAW", "32x48x128_k4_sp8_pf2_dAW",
                                              "32x96x64_w1x2_k2_sp8_pf3_il_ks2_cil_dW",
                                              "128x96x64_w2x2_sp8_pf3_il_ks8_cil_dA"};
    bool small = deep;
    for (const char *t : small_tiles) small = small || same_name(e.name, t);
    if (!small) return r;
    const int64_t cus = 256;
    const bool splits = split && K >= (ceil_div(M, 16) * ceil_div(N, 48) > cus / 2 ? 8192 : 2048);
    static const SplitCand cands[] = {
        {32, 48, 1, "32x48x128_k4_sp8_pf2_dAW"},     {32, 48, 2, "32x48x128_k4_sp8_pf2_ks2_dAW"},
        {32, 48, 4, "32x48x128_k4_sp8_pf2_ks4_dAW"}, {32, 48, 8, "32x48x128_k4_sp8_pf2_ks8_dAW"},
        {16, 48, 1, "16x48x128_k4_sp4_dAW"},         {16, 48, 2, "16x48x128_k4_sp4_ks2_dAW"},
        {16, 48, 4, "16x48x128_k4_sp4_ks4_dAW"},     {16, 48, 8, "16x48x128_k4_sp4_ks8_dAW"}};
    const char *best = pick_by_estimate(M, K, N, false, splits, 6 * cus, cands, sizeof(cands) / sizeof(cands[0]),
                                        e.name, deep ? -1.0 : split_estimate(M, K, N, false, e.bm, e.bn, e.ks));
    return table_index(kBwdConfigs, kNumBwdConfigs, best);
}

// ---------------------------------------------------------------------------
// validation + launch
// ---------------------------------------------------------------------------

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes) {
    if (a == nullptr || b == nullptr || abytes == 0 || bbytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Options of the _ex entry points, with the plain entry points' defaults.
struct Opts {
    int config = -1;
    void *ws = nullptr;
    int64_t ws_bytes = 0;
    void *start = nullptr, *stop = nullptr;
    // the workspace is the library-held array (gemm_fwd_swiglu_noalloc),
    // resolved only once the arguments have passed validation
    bool library_scratch = false;
};

int scratch_address(void **out, hipStream_t s);

int read_opts(const gemm_opts *o, int num_configs, Opts &out) {
    if (o == nullptr) return GEMM_OK;
    if (o->config < -1 || o->config >= num_configs) return GEMM_ERR_CONFIG;
    if (o->workspace_bytes < 0 || (o->workspace == nullptr && o->workspace_bytes != 0)) return GEMM_ERR_WORKSPACE;
    if (o->workspace != nullptr && !aligned(o->workspace, 256)) return GEMM_ERR_ALIGN;
    out.config = (int)o->config;
    out.ws = o->workspace;
    out.ws_bytes = o->workspace_bytes;
    out.start = o->start_event;
    out.stop = o->stop_event;
    return GEMM_OK;
}

// The configuration to launch: the explicit one, or the library's choice,
// which splits K only when the workspace holds what that needs.  Fills the
// split-K fields of p.
template <class Pick>
int resolve(const ConfigEntry *table, const Opts &o, int64_t M, int64_t N, Pick pick, Params &p, int &cfg) {
    cfg = o.config >= 0 ? o.config : pick(o.ws != nullptr);
    if (cfg < 0) return GEMM_ERR_CONFIG;
    int64_t need = split_workspace_bytes(table[cfg], M, N);
    if (need < 0) return GEMM_ERR_CONFIG;
    if (need > o.ws_bytes) {
        if (o.config >= 0) return GEMM_ERR_WORKSPACE;
        cfg = pick(false);
        if (cfg < 0) return GEMM_ERR_CONFIG;
        need = split_workspace_bytes(table[cfg], M, N);
        if (need != 0) return GEMM_ERR_CONFIG;
    }
    p.ws = nullptr;
    p.cnt = nullptr;
    p.ws_stride = M * N;
    if (need > 0) {
        p.cnt = static_cast<unsigned *>(o.ws);
        p.ws = reinterpret_cast<float *>(static_cast<char *>(o.ws) + kCounterBytes);
    }
    return GEMM_OK;
}

int run(bool swiglu, const float *A, const float *U, const void *W, bool w16, const float *R, float *Y,
        int64_t M, int64_t K, int64_t N, const Opts &o, void *stream) {
    const int64_t lim = (int64_t)1 << 31;
    if (M < 0 || K < 0 || N < 0 || M >= lim || K >= lim || N >= lim) return GEMM_ERR_SHAPE;
    // A pointer may be NULL only when its array holds no element (an empty
    // tensor has no storage); the residual of the SwiGLU variant is required.
    const bool mk = M > 0 && K > 0, kn = K > 0 && N > 0, mn = M > 0 && N > 0;
    if ((mk && A == nullptr) || (kn && W == nullptr) || (mn && Y == nullptr) ||
        (swiglu && ((mk && U == nullptr) || (mn && R == nullptr))))
        return GEMM_ERR_NULL;
    if (K % 4 != 0 || N % 4 != 0) return GEMM_ERR_SHAPE;
    // Buffer offsets are 32-bit: a tile's rows of A (up to 256 x K fp32), a
    // stage's rows of W and a tile's rows of Y (up to 256 x N fp32) must each
    // stay below 2^31 bytes.
    if (K * 1024 >= lim || N * 1024 >= lim) return GEMM_ERR_SHAPE;
    if ((A && !aligned(A, 16)) || (Y && !aligned(Y, 16)) || (U && !aligned(U, 16)) || (R && !aligned(R, 16)) ||
        (W && !aligned(W, w16 ? 8 : 16)))
        return GEMM_ERR_ALIGN;
    const size_t ybytes = (size_t)M * N * 4, abytes = (size_t)M * K * 4;
    const size_t wbytes = (size_t)K * N * (w16 ? 2 : 4);
    if (overlaps(Y, ybytes, A, abytes) || overlaps(Y, ybytes, U, abytes) ||
        overlaps(Y, ybytes, W, wbytes) || overlaps(Y, ybytes, R, ybytes))
        return GEMM_ERR_ALIAS;
    const size_t wsb = (size_t)o.ws_bytes;
    if (overlaps(o.ws, wsb, Y, ybytes) || overlaps(o.ws, wsb, A, abytes) || overlaps(o.ws, wsb, U, abytes) ||
        overlaps(o.ws, wsb, W, wbytes) || overlaps(o.ws, wsb, R, ybytes))
        return GEMM_ERR_ALIAS;
    // an explicit tile that keeps W in registers exists for fp32 W only
    if (o.config >= 0 && kConfigs[o.config].fn[swiglu ? 1 : 0][w16 ? 1 : 0][R ? 1 : 0] == nullptr)
        return GEMM_ERR_CONFIG;
    if (M == 0 || N == 0) return GEMM_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) {
        const int64_t count = M * N;
        hipExtLaunchKernelGGL(fill_k0_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, s,
                              static_cast<hipEvent_t>(o.start), static_cast<hipEvent_t>(o.stop), 0, R, Y, count);
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }

    Params p;
    int cfg = -1;
    Opts oo = o;
    if (o.library_scratch) {
        const int sa = scratch_address(&oo.ws, s);
        if (sa != GEMM_OK) return sa;
        oo.ws_bytes = kScratchBytes;
    }
    const int st = resolve(kConfigs, oo, M, N,
                           [&](bool split) { return select_config(M, K, N, swiglu, w16, split); }, p, cfg);
    if (st != GEMM_OK) return st;
    const ConfigEntry &e = kConfigs[cfg];
    p.A = A; p.U = U; p.W = W; p.R = R; p.Y = Y;
    p.EG = nullptr; p.EU = nullptr; p.Y2 = nullptr;
    p.M = (int)M; p.K = (int)K; p.N = (int)N;
    p.tiles_m = (int)ceil_div(M, e.bm);
    p.tiles_n = (int)ceil_div(N, e.bn);
    p.group_m = p.tiles_m < 4 ? p.tiles_m : 4;
    p.kchunk = (int)(ceil_div(ceil_div(K, e.ks), e.bk) * e.bk);
    const int64_t blocks = (int64_t)p.tiles_m * p.tiles_n * e.ks;
    if (blocks >= lim) return GEMM_ERR_SHAPE;
    KernelFn fn = e.fn[swiglu ? 1 : 0][w16 ? 1 : 0][R ? 1 : 0];
    if (!fn) return GEMM_ERR_CONFIG;
    // with NULL events this is a plain launch; otherwise the events take the
    // kernel's own start and end times
    hipExtLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(e.nt), 0, s, static_cast<hipEvent_t>(o.start),
                          static_cast<hipEvent_t>(o.stop), 0, p);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// The backward products (public shapes: dY [M x N], W [K x N], X / GATE / UP
// [M x K]):
//   op kOpNT, matmul_t:  dX [M x K] (+)= dY W^T   -> kernel (M, K = N, N = K)
//   op kOpTN, matmul_at: dW [K x N] (+)= A^T dY   -> kernel (M = K, K = M, N)
// with A = X, or silu(GATE) * UP.  `acc` adds the product to the output's
// current contents.
int run_bwd(int op, bool swiglu, const float *A, const float *U, const float *B, float *Y, int64_t M,
            int64_t K, int64_t N, bool acc, const Opts &o, void *stream, const float *EG = nullptr,
            const float *EU = nullptr, float *Y2 = nullptr) {
    // op kOpNT with swiglu: the fused SwiGLU backward, dGATE into Y and dUP
    // into Y2 from GATE (EG) and UP (EU), all [M x K]
    const bool fused = op == kOpNT && swiglu;
    const int64_t lim = (int64_t)1 << 31;
    if (M < 0 || K < 0 || N < 0 || M >= lim || K >= lim || N >= lim) return GEMM_ERR_SHAPE;
    const bool mk = M > 0 && K > 0, kn = K > 0 && N > 0, mn = M > 0 && N > 0;
    const bool a_null = op == kOpNT ? (mn && A == nullptr) : (mk && (A == nullptr || (swiglu && U == nullptr)));
    const bool b_null = op == kOpNT ? (kn && B == nullptr) : (mn && B == nullptr);
    const bool y_null = op == kOpNT ? (mk && Y == nullptr) : (kn && Y == nullptr);
    const bool e_null = fused && mk && (EG == nullptr || EU == nullptr || Y2 == nullptr);
    if (a_null || b_null || y_null || e_null) return GEMM_ERR_NULL;
    if (fused && acc) return GEMM_ERR_DTYPE;
    if (K % 4 != 0 || N % 4 != 0) return GEMM_ERR_SHAPE;
    if (K * 1024 >= lim || N * 1024 >= lim) return GEMM_ERR_SHAPE;
    if ((A && !aligned(A, 16)) || (U && !aligned(U, 16)) || (B && !aligned(B, 16)) || (Y && !aligned(Y, 16)) ||
        (EG && !aligned(EG, 16)) || (EU && !aligned(EU, 16)) || (Y2 && !aligned(Y2, 16)))
        return GEMM_ERR_ALIGN;
    const size_t abytes = (size_t)(op == kOpNT ? M * N : M * K) * 4;
    const size_t bbytes = (size_t)(op == kOpNT ? K * N : M * N) * 4;
    const size_t ybytes = (size_t)(op == kOpNT ? M * K : K * N) * 4;
    if (overlaps(Y, ybytes, A, abytes) || overlaps(Y, ybytes, U, abytes) || overlaps(Y, ybytes, B, bbytes))
        return GEMM_ERR_ALIAS;
    if (fused) {
        // each output may be GATE's or UP's very array (every element is read
        // before it is written, by one thread) but overlaps nothing else
        auto partial = [&](const void *o2, const void *i) { return o2 != i && overlaps(o2, ybytes, i, ybytes); };
        if (overlaps(Y2, ybytes, A, abytes) || overlaps(Y2, ybytes, B, bbytes) || overlaps(Y, ybytes, Y2, ybytes) ||
            partial(Y, EG) || partial(Y, EU) || partial(Y2, EG) || partial(Y2, EU))
            return GEMM_ERR_ALIAS;
    }
    const size_t wsb = (size_t)o.ws_bytes;
    if (overlaps(o.ws, wsb, Y, ybytes) || overlaps(o.ws, wsb, A, abytes) || overlaps(o.ws, wsb, U, abytes) ||
        overlaps(o.ws, wsb, B, bbytes) || (fused && (overlaps(o.ws, wsb, Y2, ybytes) ||
                                                     overlaps(o.ws, wsb, EG, ybytes) || overlaps(o.ws, wsb, EU, ybytes))))
        return GEMM_ERR_ALIAS;
    // kernel dimensions: output rows, contraction, output columns
    const int64_t km = op == kOpNT ? M : K, kk = op == kOpNT ? N : M, kn2 = op == kOpNT ? K : N;
    if (km == 0 || kn2 == 0) return GEMM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t e0 = static_cast<hipEvent_t>(o.start), e1 = static_cast<hipEvent_t>(o.stop);
    if (kk == 0 && fused) {
        // dH = 0: both gradients are zero
        hipExtLaunchKernelGGL(fill_k0_kernel, dim3((unsigned)ceil_div(km * kn2, 256)), dim3(256), 0, s, e0,
                              nullptr, 0, nullptr, Y, km * kn2);
        hipExtLaunchKernelGGL(fill_k0_kernel, dim3((unsigned)ceil_div(km * kn2, 256)), dim3(256), 0, s, nullptr,
                              e1, 0, nullptr, Y2, km * kn2);
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    if (kk == 0) {
        if (acc) return GEMM_OK;  // nothing to add
        const int64_t count = km * kn2;
        hipExtLaunchKernelGGL(fill_k0_kernel, dim3((unsigned)ceil_div(count, 256)), dim3(256), 0, s, e0, e1, 0,
                              nullptr, Y, count);
        return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    Params p;
    int cfg = -1;
    const int st = resolve(kBwdConfigs, o, km, kn2,
                           [&](bool split) { return select_bwd_config(op, km, kk, kn2, fused ? 0 : swiglu, split); },
                           p, cfg);
    if (st != GEMM_OK) return st;
    const ConfigEntry &e = kBwdConfigs[cfg];
    p.A = A; p.U = U; p.W = B; p.R = acc ? Y : nullptr; p.Y = Y;
    p.EG = EG; p.EU = EU; p.Y2 = Y2;
    p.M = (int)km; p.K = (int)kk; p.N = (int)kn2;
    p.tiles_m = (int)ceil_div(km, e.bm);
    p.tiles_n = (int)ceil_div(kn2, e.bn);
    p.group_m = p.tiles_m < 4 ? p.tiles_m : 4;
    p.kchunk = (int)(ceil_div(ceil_div(kk, e.ks), e.bk) * e.bk);
    const int64_t blocks = (int64_t)p.tiles_m * p.tiles_n * e.ks;
    if (blocks >= lim) return GEMM_ERR_SHAPE;
    KernelFn fn = e.fn[op == kOpTN ? 1 : 0][swiglu ? 1 : 0][acc ? 1 : 0];
    if (fn == nullptr) return GEMM_ERR_DTYPE;
    hipExtLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(e.nt), 0, s, e0, e1, 0, p);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// library-held workspace of gemm_fwd_swiglu_noalloc
// ---------------------------------------------------------------------------

// For callers that cannot allocate device memory, gemm_fwd_swiglu_noalloc
// takes its split-K workspace from this array: the counter block plus 4 MiB
// of partial slots, enough for every split the library's choice makes
// (outputs of at most 2^19 elements, K split in two).  Zero at load; every
// completed call leaves its counter block zero again.  Each GPU holds its
// own copy until the process ends.
static __device__ __align__(256) float scratch[kScratchBytes / 4];

// The device address of `scratch` on the current device, fetched once per
// device (the array's name is only a host-side stand-in in host code).  On
// the first call on a device the counter block is also cleared, by a fill
// kernel on the caller's stream.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_address(void **out, hipStream_t s) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GEMM_ERR_LAUNCH;
        hipLaunchKernelGGL(fill_k0_kernel, dim3((unsigned)ceil_div(kCounterBytes / 4, 256)), dim3(256), 0, s, nullptr,
                           static_cast<float *>(ptr), kCounterBytes / 4);
        if (hipGetLastError() != hipSuccess) return GEMM_ERR_LAUNCH;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GEMM_OK;
}

int fwd_flags(uint32_t flags, bool &w16) {
    if (flags & ~GEMM_FLAG_W_F16) return GEMM_ERR_DTYPE;
    w16 = (flags & GEMM_FLAG_W_F16) != 0;
    return GEMM_OK;
}

int bwd_flags(uint32_t flags, bool &acc) {
    if (flags & ~GEMM_FLAG_ACC) return GEMM_ERR_DTYPE;
    acc = (flags & GEMM_FLAG_ACC) != 0;
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_fwd_ex(const float *X, const void *W, const float *R, float *Y, int64_t M, int64_t K, int64_t N,
                uint32_t flags, const gemm_opts *opts, void *stream) {
    bool w16 = false;
    Opts o;
    int st = fwd_flags(flags, w16);
    if (st == GEMM_OK) st = read_opts(opts, kNumConfigs, o);
    return st != GEMM_OK ? st : run(false, X, nullptr, W, w16, R, Y, M, K, N, o, stream);
}

int gemm_fwd(const float *X, const void *W, const float *R, float *Y, int64_t M, int64_t K, int64_t N,
             uint32_t flags, void *stream) {
    return gemm_fwd_ex(X, W, R, Y, M, K, N, flags, nullptr, stream);
}

int gemm_fwd_swiglu_ex(const float *GATE, const float *UP, const void *W, const float *R, float *Y, int64_t M,
                       int64_t K, int64_t N, int w_dtype, const gemm_opts *opts, void *stream) {
    if (w_dtype != GEMM_W_F32 && w_dtype != GEMM_W_F16) return GEMM_ERR_DTYPE;
    Opts o;
    const int st = read_opts(opts, kNumConfigs, o);
    return st != GEMM_OK ? st : run(true, GATE, UP, W, w_dtype == GEMM_W_F16, R, Y, M, K, N, o, stream);
}

int gemm_fwd_swiglu(const float *GATE, const float *UP, const void *W, const float *R, float *Y, int64_t M,
                    int64_t K, int64_t N, int w_dtype, void *stream) {
    return gemm_fwd_swiglu_ex(GATE, UP, W, R, Y, M, K, N, w_dtype, nullptr, stream);
}

int gemm_fwd_swiglu_noalloc(const float *GATE, const float *UP, const void *W, const float *R, float *Y, int64_t M,
                            int64_t K, int64_t N, int w_dtype, void *stream) {
    if (w_dtype != GEMM_W_F32 && w_dtype != GEMM_W_F16) return GEMM_ERR_DTYPE;
    const int64_t need = gemm_fwd_workspace_bytes(M, K, N, 1, w_dtype == GEMM_W_F16 ? GEMM_FLAG_W_F16 : 0u, -1);
    if (need > kScratchBytes) return GEMM_ERR_WORKSPACE;   // (negative: a bad shape, reported by run)
    Opts o;
    o.library_scratch = true;
    return run(true, GATE, UP, W, w_dtype == GEMM_W_F16, R, Y, M, K, N, o, stream);
}

int64_t gemm_fwd_workspace_bytes(int64_t M, int64_t K, int64_t N, int swiglu, uint32_t flags, int config) {
    bool w16 = false;
    if (fwd_flags(flags, w16) != GEMM_OK || M < 0 || K < 0 || N < 0 || config < -1 || config >= kNumConfigs)
        return -1;
    if (M == 0 || N == 0 || K == 0) return 0;
    const int cfg = config >= 0 ? config : select_config(M, K, N, swiglu != 0, w16, true);
    return cfg < 0 ? -1 : split_workspace_bytes(kConfigs[cfg], M, N);
}

int gemm_matmul_t_ex(const float *dY, const float *W, float *dX, int64_t M, int64_t K, int64_t N, uint32_t flags,
                     const gemm_opts *opts, void *stream) {
    bool acc = false;
    Opts o;
    int st = bwd_flags(flags, acc);
    if (st == GEMM_OK) st = read_opts(opts, kNumBwdConfigs, o);
    return st != GEMM_OK ? st : run_bwd(kOpNT, false, dY, nullptr, W, dX, M, K, N, acc, o, stream);
}
int gemm_matmul_t(const float *dY, const float *W, float *dX, int64_t M, int64_t K, int64_t N, uint32_t flags,
                  void *stream) {
    return gemm_matmul_t_ex(dY, W, dX, M, K, N, flags, nullptr, stream);
}
int gemm_matmul_at_ex(const float *X, const float *dY, float *dW, int64_t M, int64_t K, int64_t N, uint32_t flags,
                      const gemm_opts *opts, void *stream) {
    bool acc = false;
    Opts o;
    int st = bwd_flags(flags, acc);
    if (st == GEMM_OK) st = read_opts(opts, kNumBwdConfigs, o);
    return st != GEMM_OK ? st : run_bwd(kOpTN, false, X, nullptr, dY, dW, M, K, N, acc, o, stream);
}
int gemm_matmul_at(const float *X, const float *dY, float *dW, int64_t M, int64_t K, int64_t N, uint32_t flags,
                   void *stream) {
    return gemm_matmul_at_ex(X, dY, dW, M, K, N, flags, nullptr, stream);
}
int gemm_matmul_at_swiglu_a_ex(const float *GATE, const float *UP, const float *dY, float *dW, int64_t M,
                               int64_t K, int64_t N, uint32_t flags, const gemm_opts *opts, void *stream) {
    bool acc = false;
    Opts o;
    int st = bwd_flags(flags, acc);
    if (st == GEMM_OK) st = read_opts(opts, kNumBwdConfigs, o);
    return st != GEMM_OK ? st : run_bwd(kOpTN, true, GATE, UP, dY, dW, M, K, N, acc, o, stream);
}
int gemm_matmul_at_swiglu_a(const float *GATE, const float *UP, const float *dY, float *dW, int64_t M, int64_t K,
                            int64_t N, uint32_t flags, void *stream) {
    return gemm_matmul_at_swiglu_a_ex(GATE, UP, dY, dW, M, K, N, flags, nullptr, stream);
}
int gemm_matmul_t_swiglu_bwd_ex(const float *dY, const float *W, const float *GATE, const float *UP, float *dGATE,
                                float *dUP, int64_t M, int64_t K, int64_t N, const gemm_opts *opts, void *stream) {
    Opts o;
    const int st = read_opts(opts, kNumBwdConfigs, o);
    return st != GEMM_OK ? st : run_bwd(kOpNT, true, dY, nullptr, W, dGATE, M, K, N, false, o, stream, GATE, UP, dUP);
}
int gemm_matmul_t_swiglu_bwd(const float *dY, const float *W, const float *GATE, const float *UP, float *dGATE,
                             float *dUP, int64_t M, int64_t K, int64_t N, void *stream) {
    return gemm_matmul_t_swiglu_bwd_ex(dY, W, GATE, UP, dGATE, dUP, M, K, N, nullptr, stream);
}

int64_t gemm_bwd_workspace_bytes(int op, int64_t M, int64_t K, int64_t N, int swiglu, int config) {
    if ((op != 1 && op != 2) || M < 0 || K < 0 || N < 0 || config < -1 || config >= kNumBwdConfigs) return -1;
    // kernel dimensions: output rows, contraction, output columns
    const int64_t km = op == 1 ? M : K, kk = op == 1 ? N : M, kn = op == 1 ? K : N;
    if (km == 0 || kn == 0 || kk == 0) return 0;
    const int cfg = config >= 0 ? config
                                : select_bwd_config(op == 1 ? kOpNT : kOpTN, km, kk, kn, op == 2 ? swiglu : 0, true);
    return cfg < 0 ? -1 : split_workspace_bytes(kBwdConfigs[cfg], km, kn);
}

int gemm_bwd_num_configs(void) { return kNumBwdConfigs; }

int gemm_bwd_select_config(int op, int64_t M, int64_t K, int64_t N, int swiglu, int with_workspace) {
    if (op == 1) return select_bwd_config(kOpNT, M, N, K, 0, with_workspace != 0);
    if (op == 2) return select_bwd_config(kOpTN, K, M, N, swiglu, with_workspace != 0);
    return -1;
}

const char *gemm_bwd_config_name(int config) {
    return (config >= 0 && config < kNumBwdConfigs) ? kBwdConfigs[config].name : nullptr;
}

int gemm_num_configs(void) { return kNumConfigs; }

const char *gemm_config_name(int config) {
    return (config >= 0 && config < kNumConfigs) ? kConfigs[config].name : nullptr;
}

int gemm_select_config(int64_t M, int64_t K, int64_t N, int swiglu, int w_f16, int with_workspace) {
    return select_config(M, K, N, swiglu, w_f16, with_workspace != 0);
}

int gemm_timing_event_create(void **event) {
    if (event == nullptr) return GEMM_ERR_NULL;
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_LAUNCH;
    }
    *event = e;
    return GEMM_OK;
}

int gemm_timing_event_record(void *event, void *stream) {
    if (event == nullptr) return GEMM_ERR_NULL;
    if (hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_LAUNCH;
    }
    return GEMM_OK;
}

int gemm_timing_elapsed_ms(void *start, void *stop, float *ms) {
    if (start == nullptr || stop == nullptr || ms == nullptr) return GEMM_ERR_NULL;
    if (hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_LAUNCH;
    }
    return GEMM_OK;
}

int gemm_timing_event_destroy(void *event) {
    if (event == nullptr) return GEMM_OK;
    if (hipEventDestroy(static_cast<hipEvent_t>(event)) != hipSuccess) {
        (void)hipGetLastError();
        return GEMM_ERR_LAUNCH;
    }
    return GEMM_OK;
}

const char *gemm_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "ok";
        case GEMM_ERR_NULL: return "a required pointer is NULL";
        case GEMM_ERR_SHAPE: return "bad shape (negative or too large, or K or N not a multiple of 4)";
        case GEMM_ERR_ALIGN: return "misaligned array (fp32 needs 16 bytes, binary16 W 8, the workspace 256)";
        case GEMM_ERR_DTYPE: return "unknown flags or weight type";
        case GEMM_ERR_ALIAS: return "an output or the workspace overlaps an input or another output";
        case GEMM_ERR_LAUNCH: return "kernel launch failed";
        case GEMM_ERR_CONFIG: return "tile configuration index out of range, or a W-in-registers tile with binary16 W";
        case GEMM_ERR_WORKSPACE: return "the workspace is missing or smaller than the configuration needs";
        default: return "unknown status";
    }
}

}  // extern "C"
