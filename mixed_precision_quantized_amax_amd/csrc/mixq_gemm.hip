// The mixed-precision GEMM: INT8 x INT8 (or INT8 x INT4) main product on
// gfx950 i8 matrix cores, FP16 outlier product on f16 matrix cores, fused
// dequantize / scale / add epilogue, one kernel.
//
// MixQ article: section "研究背景：已有量化技术总结", Fig. 5 -- the product is
// split into a low-bit part and an FP16 outlier part whose results are
// added; section "MixQ的解决方案", Fig. 12 -- the low-precision result is
// dequantized in registers and added to the high-precision one.
// QServe notes, "寄存器压力和并行性" -- keeping two sets of partial sums (one
// int32, one fp32) costs registers and occupancy; here the int32
// accumulators are converted in place once, after the K loop, and the fp32
// values then serve as the C operand of the f16 outlier MFMAs, so only one
// accumulator set is ever live.  INT4 weights are decoded to INT8 on their
// way into LDS ("小结": decode inside the main loop, all products on INT8
// units).
//
// Tiling (CDNA4, wave64):
//   block tile BM x BN, K step 64 bytes; waves arranged WM x WN, each owning
//   a (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA fragments
//   (v_mfma_i32_32x32x32_i8: 16 B of A and 16 B of B per lane, 16 int32
//   results per lane).
//   Operand tiles live in LDS as rows of 64 bytes = four 16-byte chunks;
//   chunk c of row r is stored at slot c ^ swz(r) so that both the
//   row-contiguous writes and the MFMA fragment reads (32 rows, one chunk
//   each) hit distinct banks.
//   Large products with INT8 weights use 128-byte K pairs: each global load
//   instruction covers eight rows x 128 bytes (whole L2 lines), two pair
//   buffers in LDS, two fragment register sets, and a fixed issue order that
//   spreads a phase's LDS reads, LDS writes and global loads over its MFMAs.
//   The other variants (64-byte K steps, register-staged or LDS-direct) serve
//   INT4 weights, K not a multiple of 128 and thin products.
//   Tile order: consecutive block ids go to different XCDs (round-robin), so
//   block ids are remapped to give each XCD a compact rectangle of tiles that
//   share A rows and B rows in its L2.
#include <atomic>
#include <mutex>

#include "mixq_internal.h"

namespace mixq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kBK = 64;  // bytes of K per tile: 64 int8 codes or 32 fp16 values

struct GemmArgs {
    const int8_t* Xq;
    const float* s_x;
    const uint16_t* X_out;
    const int32_t* count;
    const void* wq;
    const float* s_w;
    const uint16_t* w_out;
    int32_t ld_out;
    int32_t M, N, K;
    float* Y;
    int64_t ldy;
    int32_t* acc_debug;
    int32_t tiles_m, tiles_n;
    // this launch's output columns: tiles start at n_begin and cover
    // [n_begin, n_end) (a launch may take only part of N, see gemm_impl)
    int32_t n_begin, n_end;
    // split K (K-pair kernels): ksplit blocks per output tile, 1 or 2
    int32_t ksplit;
    int32_t* sync;  // [tiles] arrival counters, zero between calls
    int32_t* part;  // [tiles][2] int32 partial tiles
    int32_t out_mode;  // MIXQ_OUT_F32 / _F16 / _BF16, or MIXQ_OUT_SWIGLU_F16 (16-bit Y)
    // progressive INT4 (null: symmetric per-channel INT4): per row and group
    // of 128 channels, s2 | z << 8
    const uint16_t* gsz;
    // row subset (ROWS kernels): packed row -> W row = Y column, for W rows
    // in [0, n_out) (output-feature mixed precision: the 8-bit rows and the
    // 4-bit rows of one W are two such weights)
    const int32_t* rmap;
    int32_t n_out;
    int32_t wbits;  // 8 or 4 (host side: which launcher)
    // measurement hook (null: off): block b < clk_n writes its shader-clock
    // and 100 MHz real-time stamps at entry and exit to clk[4b .. 4b+3]
    int64_t* clk;
    int32_t clk_n;
};

// 64-byte rows: 16-byte piece c of row r sits at slot c ^ swz(r).  With 64
// banks of 4 bytes and 16 lanes served per pass, four rows share a bank line
// (rows r and r + 4 the same banks); swz gives the four rows of each such
// class distinct slots within any 16 consecutive rows, so fragment reads (16
// rows, one piece) and the INT4 loader's writes (8 rows, two pieces) are
// conflict-free.
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * kBK + ((c ^ swz(r)) << 4); }

// Sign-extend eight 4-bit codes held as the low nibbles of four bytes.
__device__ __forceinline__ uint32_t sext_nibbles(uint32_t v) {
    const uint32_t s = v & 0x08080808u;
    return v | ((s << 5) - (s << 1));  // s * 0x1E: 0x08 -> 0xF0 per byte, no carries
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Progressive INT4 (QServe page, progressive group quantization): the
// rebuilt INT8 code (u - z) * s2 of four 4-bit values u (one per byte),
// computed as u * s2 + (128 - z * s2) in 16-bit lanes -- no carries between
// lanes; the result is the code plus 128, in [0, 255] -- and turned back into
// two's complement by flipping each byte's top bit.
__device__ __forceinline__ uint32_t prog_decode4(uint32_t u4, u16x2 s2v, u16x2 cv) {
    const u16x2 e = __builtin_bit_cast(u16x2, u4 & 0x00FF00FFu);
    const u16x2 o = __builtin_bit_cast(u16x2, (u4 >> 8) & 0x00FF00FFu);
    const uint32_t re = __builtin_bit_cast(uint32_t, e * s2v + cv);
    const uint32_t ro = __builtin_bit_cast(uint32_t, o * s2v + cv);
    return (re | (ro << 8)) ^ 0x80808080u;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over [base, base + bytes): loads past the end return 0,
// which covers the ragged last tile rows without clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (<= n, n < 64).
#define MIXQ_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8)))

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer descriptor as four dwords (base, stride 0, size in bytes, the
// flags make_rsrc uses), for loads issued from inline assembly.
__device__ __forceinline__ v4u rsrc_words(const void* base, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const unsigned n = bytes > 0x7FFFFFFF ? 0x7FFFFFFFu : (unsigned)bytes;
    return v4u{(unsigned)b, (unsigned)(b >> 32) & 0xFFFFu, n, 0x00020000u};
}

// One 16-byte-per-lane load straight into LDS (lane l's bytes at lds + 16 l),
// issued from inline assembly so that the compiler's wait insertion does not
// see it (inside a loop it cannot tell such a transfer's target from the
// buffers the loop reads, and would wait for it before every LDS read).  The
// caller waits for it with the vector-memory counter before reading the
// target, and keeps every wave from leaving with it in flight.  No register
// receives data; the offset, descriptor and LDS address (M0: one wait state
// before the load, restored after it) are read when the instruction issues.
__device__ __forceinline__ void lds_load16(const v4u& rsrc, uint32_t lds, int voff, int soff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory");
}

// Scheduling pattern for one pipelined tile: the first MFMAs each followed by
// an LDS write or a global load (so the loads issue early and have the whole
// tile to land), the next ones each followed by LDS reads of the next tile's
// fragments, then the rest (sched_group_barrier masks: 0x008 MFMA, 0x100 LDS
// read, 0x200 LDS write, 0x020 global load).
template <int MF, int RD, int WR, int LD>
__device__ __forceinline__ void sched_interleave();
// The order the pinned K-pair loop settled on, as a pattern for the
// compiler: the MFMAs first each followed by one LDS read, then each by one
// LDS write or global load, so that the LDS writes are spread over as many
// MFMAs as they number and come after the reads.  (Symmetric INT4 prefill
// GEMM: 117.6-118.4 us against 119.8-120.2 us with sched_interleave's order,
// results identical.)  A phase with more memory instructions than MFMAs
// takes sched_interleave's pattern.
template <int MF, int RD, int WR, int LD>
__device__ __forceinline__ void sched_reads_first() {
    if constexpr (RD + WR + LD > MF) {
        sched_interleave<MF, RD, WR, LD>();
    } else {
#pragma unroll
        for (int i = 0; i < RD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < WR + LD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x220, 1, 0);
        }
        if constexpr (MF - RD - WR - LD > 0)
            __builtin_amdgcn_sched_group_barrier(0x008, MF - RD - WR - LD, 0);
    }
}
template <int MF, int RD, int WR, int LD>
__device__ __forceinline__ void sched_interleave() {
    constexpr int H = (WR + LD) < MF / 2 ? (WR + LD) : MF / 2;
    constexpr int opm = (WR + LD + H - 1) / H;
    constexpr int R = MF - H;
    constexpr int rpm = (RD + R - 1) / R;
#pragma unroll
    for (int i = 0; i < H; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x220, opm, 0);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, rpm, 0);
    }
}

template <int BM, int BN, int WM, int WN, int BITS>
struct Cfg {
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kNW = WM * WN;
    static constexpr int kWTM = BM / WM;
    static constexpr int kWTN = BN / WN;
    static constexpr int kFM = kWTM / 32;
    static constexpr int kFN = kWTN / 32;
    // one load instruction of a wave fills 16 rows x 64 B (int8 / fp16 rows)
    static constexpr int kAI = BM / 16 / kNW;
    static constexpr int kBI = BN / 16 / kNW;
    // packed INT4 rows: 32 rows x 32 B per wave instruction
    static constexpr int kBI4 = BN / 32 / kNW;
    static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "tile/wave mismatch");
    static_assert(BM % (16 * kNW) == 0 && BN % (32 * kNW) == 0, "loader mismatch");
};

// STAGES == 2: global -> VGPR -> LDS, two 64-byte K tile buffers.
// STAGES == 4: the K-pair loaders (PF 5 and 6): two pair buffers of 128-byte
// rows, held as four arrays.
// Large tiles hold 256 int32 accumulators per lane, so one wave per SIMD is
// all that fits; saying so lets the scheduler spend registers on overlapping
// LDS reads with MFMAs instead of saving them for an occupancy it cannot get.
template <int BM, int BN, int WM, int WN>
constexpr int waves_per_eu() {
    return (BM / WM) * (BN / WN) >= 128 * 128 ? 1 : 2;
}

// PROG: progressive group-wise INT4 weights (a compile-time choice: a
// branch in the loader would split the interleaved main loop).
template <int BM, int BN, int WM, int WN, int BITS, int STAGES, int PF, bool DEBUG,
          bool PROG = false, bool ROWS = false>
__global__ __launch_bounds__(WM* WN* kWave)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<BM, BN, WM, WN>(), waves_per_eu<BM, BN, WM, WN>())))
void gemm_kernel(GemmArgs a) {
    using C = Cfg<BM, BN, WM, WN, BITS>;
    static_assert(!PROG || BITS == 4, "progressive groups are INT4");
    static_assert(STAGES == 2 || (STAGES == 4 && (PF == 5 || PF == 6)), "loader / stages");
    static_assert(PF == 1 || PF == 4 || PF == 5 || PF == 6, "loader variant");
    // One array per stage (A tile, then B tile): the compiler then tracks each
    // stage's pending global->LDS transfers separately and waits only for the
    // right ones.
    constexpr int kStageBytes = (BM + BN) * kBK;
    __shared__ __attribute__((aligned(1024))) uint8_t sS0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sS1[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sS2[STAGES == 4 ? kStageBytes : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t sS3[STAGES == 4 ? kStageBytes : 16];
    uint8_t* const sA0 = sS0;
    uint8_t* const sA1 = sS1;
    uint8_t* const sB0 = sS0 + BM * kBK;
    uint8_t* const sB1 = sS1 + BM * kBK;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / WN, wn = wave % WN;
    // size of the outlier set (read once, long before the epilogue needs it)
    const int count = *a.count;
    const int nchunks = (count + MIXQ_OUTLIER_ALIGN - 1) / MIXQ_OUTLIER_ALIGN;  // 32 columns each
    const int ldb = a.ld_out * 2;  // bytes per outlier row
    // Outlier chunks already in flight when the epilogue starts (K-pair
    // kernels load the first two into the pair buffer the K loop frees
    // first), and that buffer (0: stage arrays 0 and 1, 1: arrays 2 and 3).
    int pre = 0, cf = 0;
    int64_t clk_t0 = 0, clk_r0 = 0;
    if (a.clk) {
        clk_t0 = (int64_t)__builtin_amdgcn_s_memtime();
        clk_r0 = (int64_t)__builtin_amdgcn_s_memrealtime();
    }
    auto clk_end = [&]() __attribute__((always_inline)) {
        if (a.clk && tid == 0 && (int)blockIdx.x < a.clk_n) {
            const int64_t t1 = (int64_t)__builtin_amdgcn_s_memtime();
            const int64_t r1 = (int64_t)__builtin_amdgcn_s_memrealtime();
            int64_t* c = a.clk + 4 * (int64_t)blockIdx.x;
            c[0] = clk_t0;
            c[1] = t1;
            c[2] = clk_r0;
            c[3] = r1;
        }
    };

    // ---- block id -> tile, XCD-aware ------------------------------------------
    int bid = blockIdx.x;
    const int T = gridDim.x;
    if ((T & 7) == 0) bid = (bid & 7) * (T >> 3) + (bid >> 3);
    // the split blocks of a tile are consecutive ids (the same XCD after the remap)
    const int split = bid % a.ksplit;
    const int tbid = bid / a.ksplit;
    const int gm = a.tiles_m < 8 ? a.tiles_m : 8;
    const int group = tbid / (gm * a.tiles_n);
    const int first_m = group * gm;
    const int gsize = min(gm, a.tiles_m - first_m);
    const int within = tbid - group * gm * a.tiles_n;
    const int tm = first_m + within % gsize;
    const int tn = within / gsize;
    const int m0 = tm * BM, n0 = a.n_begin + tn * BN;

    const int K = a.K;
    const int KT = K / kBK;
    const int rows_a = min(BM, a.M - m0);
    const int rows_b = min(BN, a.N - n0);
    const int wrow_bytes = BITS == 8 ? K : K / 2;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(a.Xq + (int64_t)m0 * K, (int64_t)rows_a * K);
    // INT4 rows are stored in whole 32-row blocks (the tile's rows start on one)
    const __amdgpu_buffer_rsrc_t rB =
        make_rsrc(static_cast<const uint8_t*>(a.wq) + (int64_t)n0 * wrow_bytes,
                  (int64_t)(BITS == 8 ? rows_b : (rows_b + 31) / 32 * 32) * wrow_bytes);

    // ---- the tile's scales, staged in LDS by transfers issued now -----------------
    // Every loader waits for its first operand loads before its first LDS
    // write, which (loads complete in order) covers these earlier transfers,
    // and the barrier after it makes each wave's share visible; the epilogue
    // reads them with no wait of its own.  Rows past M or N read zero (buffer
    // range check); their outputs are never stored.
    __shared__ __attribute__((aligned(16))) float sx_t[BM];
    __shared__ __attribute__((aligned(16))) float sw_t[BN];
    {
        [[maybe_unused]] const __amdgpu_buffer_rsrc_t rSx = make_rsrc(a.s_x + m0, (int64_t)rows_a * 4);
        [[maybe_unused]] const __amdgpu_buffer_rsrc_t rSw = make_rsrc(a.s_w + n0, (int64_t)rows_b * 4);
#if defined(__HIP_DEVICE_COMPILE__)  // LDS address-space casts exist only in the device pass
        // one wave instruction stages 64 consecutive scales
        for (int q = wave; q < BM / kWave; q += C::kNW)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSx, (lds_ptr_t)(sx_t + q * kWave), 4,
                                                     lane * 4, q * kWave * 4, 0, 0);
        for (int q = wave; q < BN / kWave; q += C::kNW)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSw, (lds_ptr_t)(sw_t + q * kWave), 4,
                                                     lane * 4, q * kWave * 4, 0, 0);
#endif
    }

    // ---- per-lane load slots ------------------------------------------------------
    // Wave instruction i fills rows R0..R0+15 (R0 = (i*NW + wave)*16); lane l
    // writes LDS bytes R0*64 + 16*l, i.e. row R0 + l/4, slot l%4, which holds
    // chunk (l%4) ^ swz(row) of that row.
    int voffA[C::kAI], voffB[C::kBI];
#pragma unroll
    for (int i = 0; i < C::kAI; ++i) {
        const int row = (i * C::kNW + wave) * 16 + (lane >> 2);
        voffA[i] = row * K + (((lane & 3) ^ swz(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < C::kBI; ++i) {
        const int row = (i * C::kNW + wave) * 16 + (lane >> 2);
        voffB[i] = row * K + (((lane & 3) ^ swz(row)) << 4);
    }
    // INT4: wave instruction i covers packed rows R0..R0+31 (R0 = 32 (i NW +
    // wave), one 32-row block of the K-tile-major layout), lane -> row R0 +
    // l/2, half l%2: the instruction reads the block's 1 KiB for one K tile
    int voffB4[C::kBI4];
#pragma unroll
    for (int i = 0; i < C::kBI4; ++i) voffB4[i] = (i * C::kNW + wave) * KT * 1024 + lane * 16;

    // ---- per-lane fragment read offsets (bytes within a stage) ------------------------
    const int fr = lane & 31;
    const int fh = lane >> 5;
    int rdA[2], rdB[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        rdA[ks] = (wm * C::kWTM + fr) * kBK + (((2 * ks + fh) ^ swz(fr)) << 4);
        rdB[ks] = (wn * C::kWTN + fr) * kBK + (((2 * ks + fh) ^ swz(fr)) << 4);
    }

    v16i acc[C::kFM][C::kFN];
#pragma unroll
    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
        for (int j = 0; j < C::kFN; ++j) acc[i][j] = v16i{};

    // One K tile: both 32-byte K halves' fragments are read from LDS up
    // front, so the second half's reads overlap the first half's MFMAs.
    auto mma_tile = [&](const uint8_t* Ab, const uint8_t* Bb) {
        v4i af[2][C::kFM], bf[2][C::kFN];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int j = 0; j < C::kFN; ++j)
                bf[ks][j] = *reinterpret_cast<const v4i*>(Bb + rdB[ks] + j * 32 * kBK);
#pragma unroll
            for (int i = 0; i < C::kFM; ++i)
                af[ks][i] = *reinterpret_cast<const v4i*>(Ab + rdA[ks] + i * 32 * kBK);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < C::kFM; ++i)
#pragma unroll
                for (int j = 0; j < C::kFN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks][i], bf[ks][j],
                                                                      acc[i][j], 0, 0, 0);
        // schedule: the first half's reads, the second half's reads, then the
        // MFMAs (the second half's reads land while the first half multiplies)
        __builtin_amdgcn_sched_group_barrier(0x100, C::kFM + C::kFN, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, C::kFM + C::kFN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::kFM * C::kFN, 0);
    };

    if constexpr (PF == 5 || PF == 6) {
        // ---- 128-byte K pairs, register-staged ------------------------------------------
        // Global loads fetch 128 bytes of K per row (eight lanes per row),
        // i.e. whole L2 lines: with 64-byte row pieces every request moves
        // half a line and the L2 delivers markedly fewer bytes per clock.
        // LDS holds two pair buffers, each A[BM][128] + B[BN][128]; chunk c of
        // row r sits at slot c ^ ((r >> 1) & 7).  gfx950's LDS serves a
        // 16-byte read for 16 lanes at a time from 64 banks of 4 bytes, so a
        // 256-byte bank line holds two 128-byte rows (even rows in one half,
        // odd rows in the other); the 16 rows of a fragment read's lane group
        // then fall on 16 distinct bank quads, and the linear per-lane writes
        // are conflict-free as well.  (The swizzle c ^ (r & 7), conflict-free
        // for 32 banks, put rows r and r + 8 on the same banks: the counters
        // showed a bank-conflict cycle for every two LDS instructions.)
        // Tiles (64 bytes of K) alternate between two fragment register sets:
        //   phase A of pair p: MFMAs of tile 2p; read tile 2p+1 (pair p, upper
        //     half); write pair p+1's B rows; load pair p+2's B rows; barrier.
        //   phase B of pair p: MFMAs of tile 2p+1; read tile 2p+2 (pair p+1,
        //     lower half); write pair p+2's A rows; load pair p+3's A rows.
        // Every load has two phases to land, each phase carries the same mix
        // of MFMAs, LDS reads, LDS writes and global loads, and the one
        // barrier per pair orders all buffer reuse: a pair buffer is rewritten
        // only after the barrier that follows the last read of its previous
        // pair.
        static_assert(BITS == 8 && STAGES == 4, "pair loader: int8 operands, four 32 KiB arrays");
        constexpr int kPR = 2 * kBK;           // LDS row bytes
        constexpr int kPI = BM / 8 / C::kNW;   // load instructions per operand per wave
        static_assert(BM == BN && BM * kPR == kStageBytes, "pair buffer = one stage array");
        auto PA = [&](int c) { return c ? sS2 : sS0; };
        auto PB = [&](int c) { return c ? sS3 : sS1; };
        // this block's K range: pairs pb .. pb + KP - 1
        const int KP = K / kPR / a.ksplit;
        const int pb = split * KP;
        // load lane -> row (i*NW + wave)*8 + lane/8, LDS slot lane%8, holding
        // chunk (lane%8) ^ ((row >> 1) & 7); the LDS write of a wave
        // instruction is linear
        const int lr = lane >> 3, ls = lane & 7;
        int voff[kPI];
#pragma unroll
        for (int i = 0; i < kPI; ++i) {
            const int row = (i * C::kNW + wave) * 8 + lr;
            voff[i] = row * K + ((ls ^ ((row >> 1) & 7)) << 4);
        }
        const int wr = wave * 8 * kPR + lane * 16;  // + i * NW * 8 * kPR
        // fragment reads: tile half h, K half ks -> chunk 4h + 2ks + fh of row
        // r, (r >> 1) & 7 == (fr >> 1) & 7 (fragment rows start on multiples of 32)
        int rdA2[2][2], rdB2[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int sl = ((4 * h + 2 * ks + fh) ^ ((fr >> 1) & 7)) << 4;
                rdA2[h][ks] = (wm * C::kWTM + fr) * kPR + sl;
                rdB2[h][ks] = (wn * C::kWTN + fr) * kPR + sl;
            }
        typedef v4i Stg[kPI];
        typedef v4i AFr[2][C::kFM];
        typedef v4i BFr[2][C::kFN];
        // Pair offsets go into the per-lane offset, which the buffer range
        // check covers: loads of rows past the tile's last row read zeros.
        auto gload = [&](const __amdgpu_buffer_rsrc_t& r, int p, Stg& S) {
#pragma unroll
            for (int i = 0; i < kPI; ++i)
                S[i] = __builtin_amdgcn_raw_buffer_load_b128(r, voff[i] + (pb + p) * kPR, 0, 0);
        };
        auto lstore = [&](const Stg& S, uint8_t* buf) {
#pragma unroll
            for (int i = 0; i < kPI; ++i)
                *reinterpret_cast<v4i*>(&buf[wr + i * C::kNW * 8 * kPR]) = S[i];
        };
        auto lread = [&](const uint8_t* Ab, const uint8_t* Bb, int h, AFr& fa, BFr& fb) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int i = 0; i < C::kFM; ++i)
                    fa[ks][i] = *reinterpret_cast<const v4i*>(Ab + rdA2[h][ks] + i * 32 * kPR);
#pragma unroll
                for (int j = 0; j < C::kFN; ++j)
                    fb[ks][j] = *reinterpret_cast<const v4i*>(Bb + rdB2[h][ks] + j * 32 * kPR);
            }
        };
        auto mfmas = [&](const AFr& fa, const BFr& fb) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < C::kFM; ++i)
#pragma unroll
                    for (int j = 0; j < C::kFN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[ks][i], fb[ks][j],
                                                                          acc[i][j], 0, 0, 0);
        };
        AFr fa0, fa1;
        BFr fb0, fb1;
        Stg SA, SB;
        // prologue: pair 0 to LDS, tile 0 to registers, pair 1's A rows to
        // LDS, loads of pair 1's B rows and pair 2's A rows in flight.  No
        // conditions, so that the loop is entered with the same loads in
        // flight, in the same order, on every path and its waits count
        // exactly; for K < 384 the extra loads fetch bytes past the row's end,
        // from the next row (or zeros past the buffer), which are never read.
        gload(rA, 0, SA);
        gload(rB, 0, SB);
        lstore(SA, PA(0));
        lstore(SB, PB(0));
        gload(rA, 1, SA);
        gload(rB, 1, SB);
        __syncthreads();
        lread(PA(0), PB(0), 0, fa0, fb0);
        lstore(SA, PA(1));
        gload(rA, 2, SA);
        int p = 0;
        // Outlier chunk j (j < 2) of both tiles into array j of pair buffer
        // b, laid out as the epilogue's stage arrays (a 64-byte K tile: row
        // r's 16-byte piece q at slot q ^ swz(r)).
        auto prefetch_outliers = [&](int b, int nch) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
            const v4u wXo = rsrc_words(reinterpret_cast<const uint8_t*>(a.X_out) + (int64_t)m0 * ldb,
                                       (int64_t)rows_a * ldb);
            const v4u wWo = rsrc_words(reinterpret_cast<const uint8_t*>(a.w_out) + (int64_t)n0 * ldb,
                                       (int64_t)rows_b * ldb);
            for (int j = 0; j < nch; ++j) {
                const uint32_t stg = (uint32_t)(uintptr_t)(lds_ptr_t)(j == 0 ? PA(b) : PB(b));
#pragma unroll
                for (int i = 0; i < C::kAI; ++i) {
                    const int row = (i * C::kNW + wave) * 16 + (lane >> 2);
                    lds_load16(wXo, stg + ((i * C::kNW + wave) * 16) * kBK,
                               row * ldb + (((lane & 3) ^ swz(row)) << 4), j * kBK);
                }
#pragma unroll
                for (int i = 0; i < C::kBI; ++i) {
                    const int row = (i * C::kNW + wave) * 16 + (lane >> 2);
                    lds_load16(wWo, stg + BM * kBK + ((i * C::kNW + wave) * 16) * kBK,
                               row * ldb + (((lane & 3) ^ swz(row)) << 4), j * kBK);
                }
            }
#endif
        };
        // steady state: every load, write and read of the pair exists
        if constexpr (PF == 6) {
            // Issue order pinned slot by slot (the scheduler may not move
            // anything across a slot): each of a phase's 32 MFMAs is followed
            // by at most one memory instruction.  The first 16 carry the LDS
            // reads (their results are needed right after the phase); the
            // other 16 alternate the 8 LDS writes and the 8 global loads, the
            // load that refills a staging register one slot after the write
            // that empties it.  A wave's 16-byte-per-lane LDS write moves
            // 1 KiB; spread over 16 slots instead of 8 consecutive ones
            // (each with its load), the writes no longer hold up the MFMA
            // issue: 1.5-2% less time per launch at the prefill shape, three
            // boxes, alternating builds, results identical.
            constexpr int kMF = 2 * C::kFM * C::kFN;   // 32 MFMAs per phase
            constexpr int kRD = 2 * (C::kFM + C::kFN); // 16 fragment reads
            static_assert(kMF == 32 && kRD == 16 && kPI == 8, "slot plan for 128x128 waves");
            auto mf = [&](const AFr& fa, const BFr& fb, int t) {
                const int ks = t >> 4, i = (t >> 2) & 3, j = t & 3;
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[ks][i], fb[ks][j], acc[i][j],
                                                                  0, 0, 0);
            };
            auto rd = [&](const uint8_t* Ab, const uint8_t* Bb, int h, AFr& fa, BFr& fb, int r) {
                const int ks = r >> 3, q = r & 7;
                if (q < 4)
                    fa[ks][q] = *reinterpret_cast<const v4i*>(Ab + rdA2[h][ks] + q * 32 * kPR);
                else
                    fb[ks][q - 4] =
                        *reinterpret_cast<const v4i*>(Bb + rdB2[h][ks] + (q - 4) * 32 * kPR);
            };
            // staging register w to LDS, and its refill with pair pl's rows
            auto wo = [&](const Stg& S, uint8_t* buf, int w) {
                *reinterpret_cast<v4i*>(&buf[wr + w * C::kNW * 8 * kPR]) = S[w];
            };
            auto lo = [&](Stg& S, const __amdgpu_buffer_rsrc_t& r, int pl, int w) {
                S[w] = __builtin_amdgcn_raw_buffer_load_b128(r, voff[w] + (pb + pl) * kPR, 0, 0);
            };
            for (; p + 3 < KP; ++p) {
                const int c = p & 1, n = c ^ 1;
#pragma unroll
                for (int t = 0; t < kMF; ++t) {
                    mf(fa0, fb0, t);
                    if (t < kRD) rd(PA(c), PB(c), 1, fa1, fb1, t);
                    else if (t % 2 == 0) wo(SB, PB(n), (t - kRD) / 2);
                    else lo(SB, rB, p + 2, (t - kRD) / 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
                __syncthreads();
#pragma unroll
                for (int t = 0; t < kMF; ++t) {
                    mf(fa1, fb1, t);
                    if (t < kRD) rd(PA(n), PB(n), 0, fa0, fb0, t);
                    else if (t % 2 == 0) wo(SA, PA(c), (t - kRD) / 2);
                    else lo(SA, rA, p + 3, (t - kRD) / 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // The last three pairs, pinned the same way with their
            // conditions resolved: no global load past the last pair, no LDS
            // write past it, and the outlier prefetch after the middle pair's
            // first phase.  (Left to the general loop below, whose branches
            // split the schedule into blocks, they took 4.3 kcycles per pair
            // against 2.3 in the steady loop.)
            if (KP >= 3) {
                {  // pair KP - 3
                    const int c = p & 1, n = c ^ 1;
#pragma unroll
                    for (int t = 0; t < kMF; ++t) {
                        mf(fa0, fb0, t);
                        if (t < kRD) rd(PA(c), PB(c), 1, fa1, fb1, t);
                        else if (t % 2 == 0) wo(SB, PB(n), (t - kRD) / 2);
                        else lo(SB, rB, p + 2, (t - kRD) / 2);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    __syncthreads();
#pragma unroll
                    for (int t = 0; t < kMF; ++t) {
                        mf(fa1, fb1, t);
                        if (t < kRD) rd(PA(n), PB(n), 0, fa0, fb0, t);
                        else if (t % 2 == 0) wo(SA, PA(c), (t - kRD) / 2);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    ++p;
                }
                {  // pair KP - 2
                    const int c = p & 1, n = c ^ 1;
#pragma unroll
                    for (int t = 0; t < kMF; ++t) {
                        mf(fa0, fb0, t);
                        if (t < kRD) rd(PA(c), PB(c), 1, fa1, fb1, t);
                        else if (t % 2 == 0) wo(SB, PB(n), (t - kRD) / 2);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    __syncthreads();
                    if (a.ksplit == 1 && nchunks > 0) {
                        // pair KP - 2's buffer is free from here on (see below)
                        pre = min(2, nchunks);
                        cf = c;
                        prefetch_outliers(c, pre);
                    }
#pragma unroll
                    for (int t = 0; t < kMF; ++t) {
                        mf(fa1, fb1, t);
                        if (t < kRD) rd(PA(n), PB(n), 0, fa0, fb0, t);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    ++p;
                }
                {  // pair KP - 1
                    const int c = p & 1;
#pragma unroll
                    for (int t = 0; t < kMF; ++t) {
                        mf(fa0, fb0, t);
                        if (t < kRD) rd(PA(c), PB(c), 1, fa1, fb1, t);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    __syncthreads();
#pragma unroll
                    for (int t = 0; t < kMF; ++t) {
                        mf(fa1, fb1, t);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    ++p;
                }
            }
        } else {
            for (; p + 3 < KP; ++p) {
                const int c = p & 1, n = c ^ 1;
                lread(PA(c), PB(c), 1, fa1, fb1);
                mfmas(fa0, fb0);
                lstore(SB, PB(n));
                gload(rB, p + 2, SB);
                sched_interleave<2 * C::kFM * C::kFN, 2 * (C::kFM + C::kFN), kPI, kPI>();
                __syncthreads();
                lread(PA(n), PB(n), 0, fa0, fb0);
                mfmas(fa1, fb1);
                lstore(SA, PA(c));
                gload(rA, p + 3, SA);
                sched_interleave<2 * C::kFM * C::kFN, 2 * (C::kFM + C::kFN), kPI, kPI>();
            }
        }
        // last pairs
        for (; p < KP; ++p) {
            const int c = p & 1, n = c ^ 1;
            lread(PA(c), PB(c), 1, fa1, fb1);
            mfmas(fa0, fb0);
            if (p + 1 < KP) lstore(SB, PB(n));
            if (p + 2 < KP) gload(rB, p + 2, SB);
            __syncthreads();
            if (p == KP - 2 && a.ksplit == 1 && nchunks > 0) {
                // Pair p's buffer is free from here on (this phase read its
                // last fragments, and no later pair is stored into it): the
                // first outlier chunks load into it while the last one and a
                // half pairs multiply, instead of after the loop.  The
                // epilogue waits for them with its other outlier loads.
                pre = min(2, nchunks);
                cf = c;
                prefetch_outliers(c, pre);
            }
            if (p + 1 < KP) lread(PA(n), PB(n), 0, fa0, fb0);
            mfmas(fa1, fb1);
            if (p + 2 < KP) lstore(SA, PA(c));
            if (p + 3 < KP) gload(rA, p + 3, SA);
        }
        __syncthreads();
    } else if constexpr (STAGES == 2) {
        // ---- register-staged, double-buffered LDS ------------------------------------
        // Global loads run PF tiles ahead of the multiply, in PF register sets.
        struct Regs {
            v4i a[C::kAI];
            v4i b[BITS == 8 ? C::kBI : C::kBI4];
            uint32_t g[PROG ? C::kBI4 : 1];  // progressive INT4: the rows' s2 | z << 8
        };
        // progressive INT4: groups of 128 channels = two K tiles; the table is
        // group-major ([K/128][N]), so one group's entries of a wave's 32 rows
        // are one contiguous 64-byte run
        const int ngroups = K / 128;
        const __amdgpu_buffer_rsrc_t rG =
            make_rsrc(a.gsz + n0,
                      a.gsz ? ((int64_t)(ngroups - 1) * a.N + rows_b) * 2 : 0);
        auto gzload = [&](int kt, Regs& R) {
            if constexpr (PROG) {
#pragma unroll
                for (int i = 0; i < C::kBI4; ++i) {
                    const int row = (i * C::kNW + wave) * 32 + (lane >> 1);
                    R.g[i] = __builtin_amdgcn_raw_buffer_load_b16(rG, ((kt / 2) * a.N + row) * 2,
                                                                   0, 0);
                }
            }
        };
        // INT4 -> INT8 codes of one staged 16-byte load: symmetric codes are
        // sign-extended nibbles, progressive ones are rebuilt from u, s2, z
        auto decode4 = [&](const Regs& R, int i, v4i& lo, v4i& hi) {
            const uint32_t w[4] = {(uint32_t)R.b[i][0], (uint32_t)R.b[i][1], (uint32_t)R.b[i][2],
                                   (uint32_t)R.b[i][3]};
            if constexpr (PROG) {
                const uint32_t g = R.g[i];
                const unsigned short s2 = g & 0xFFu;
                const unsigned short c = (unsigned short)(128u - (g >> 8) * s2);
                const u16x2 s2v = {s2, s2}, cv = {c, c};
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    lo[2 * q] = (int)prog_decode4(w[q] & 0x0F0F0F0Fu, s2v, cv);
                    lo[2 * q + 1] = (int)prog_decode4((w[q] >> 4) & 0x0F0F0F0Fu, s2v, cv);
                    hi[2 * q] = (int)prog_decode4(w[2 + q] & 0x0F0F0F0Fu, s2v, cv);
                    hi[2 * q + 1] = (int)prog_decode4((w[2 + q] >> 4) & 0x0F0F0F0Fu, s2v, cv);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    lo[2 * q] = (int)sext_nibbles(w[q] & 0x0F0F0F0Fu);
                    lo[2 * q + 1] = (int)sext_nibbles((w[q] >> 4) & 0x0F0F0F0Fu);
                    hi[2 * q] = (int)sext_nibbles(w[2 + q] & 0x0F0F0F0Fu);
                    hi[2 * q + 1] = (int)sext_nibbles((w[2 + q] >> 4) & 0x0F0F0F0Fu);
                }
            }
        };
        auto gload = [&](int kt, Regs& R) {
#pragma unroll
            for (int i = 0; i < C::kAI; ++i)
                R.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, voffA[i], kt * kBK, 0);
            if constexpr (BITS == 8) {
#pragma unroll
                for (int i = 0; i < C::kBI; ++i)
                    R.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, voffB[i], kt * kBK, 0);
            } else {
#pragma unroll
                for (int i = 0; i < C::kBI4; ++i)
                    R.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, voffB4[i], kt * 1024, 0);
                gzload(kt, R);
            }
        };
        auto lstore = [&](const Regs& R, int buf) {
            uint8_t* Ab = buf ? sA1 : sA0;
            uint8_t* Bb = buf ? sB1 : sB0;
#pragma unroll
            for (int i = 0; i < C::kAI; ++i)
                *reinterpret_cast<v4i*>(&Ab[((i * C::kNW + wave) * 16) * kBK + lane * 16]) = R.a[i];
            if constexpr (BITS == 8) {
#pragma unroll
                for (int i = 0; i < C::kBI; ++i)
                    *reinterpret_cast<v4i*>(&Bb[((i * C::kNW + wave) * 16) * kBK + lane * 16]) =
                        R.b[i];
            } else {
#pragma unroll
                for (int i = 0; i < C::kBI4; ++i) {
                    const int row = (i * C::kNW + wave) * 32 + (lane >> 1);
                    const int c2 = lane & 1;
                    v4i lo, hi;
                    decode4(R, i, lo, hi);
                    *reinterpret_cast<v4i*>(&Bb[lds_off(row, 2 * c2)]) = lo;
                    *reinterpret_cast<v4i*>(&Bb[lds_off(row, 2 * c2 + 1)]) = hi;
                }
            }
        };
        if constexpr (PF == 4) {
            // Cross-tile software pipeline.  Iteration k multiplies tile k from
            // fragments already in registers while it (a) reads tile k+1's
            // fragments from LDS, (b) writes tile k+2 (staged in registers two
            // iterations earlier) into the LDS buffer tile k used, and (c)
            // loads tile k+4 from global memory into the freed staging
            // registers.  One barrier per iteration; the MFMA pipe never waits
            // for an LDS read issued in the same iteration.
            typedef v4i AFr[2][C::kFM];
            typedef v4i BFr[2][C::kFN];
            auto lread = [&](const uint8_t* Ab, const uint8_t* Bb, AFr& fa, BFr& fb) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int i = 0; i < C::kFM; ++i)
                        fa[ks][i] = *reinterpret_cast<const v4i*>(Ab + rdA[ks] + i * 32 * kBK);
#pragma unroll
                    for (int j = 0; j < C::kFN; ++j)
                        fb[ks][j] = *reinterpret_cast<const v4i*>(Bb + rdB[ks] + j * 32 * kBK);
                }
            };
            auto mfmas = [&](const AFr& fa, const BFr& fb) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
                        for (int j = 0; j < C::kFN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
            };
            AFr fa0, fa1;
            BFr fb0, fb1;
            Regs S0, S1;
            // this block's K tiles kb .. kb + KTs - 1 (a split K range on
            // 128 x 128 tiles; the host keeps each range a whole number of
            // 128-channel groups)
            const int KTs = BM == kSplitTile ? KT / a.ksplit : KT;
            const int kb = BM == kSplitTile ? split * KTs : 0;
            gload(kb, S0);
            gload(kb + 1, S1);
            lstore(S0, 0);
            lstore(S1, 1);
            // Same issue order as the loop (S0's tile before S1's), and no
            // condition: every path into the loop then has S1's loads newest,
            // so the waits derived at the loop head leave them in flight.  For
            // KTs < 4 the extra loads read past the block's K range (the next
            // range, or the next row), which stays inside the buffer (or reads
            // zeros past its end) and is unused.
            __builtin_amdgcn_sched_barrier(0);
            gload(kb + 2, S0);
            __builtin_amdgcn_sched_barrier(0);
            gload(kb + 3, S1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            lread(sA0, sB0, fa0, fb0);
            __syncthreads();
            int k = 0;
            // Issue pattern of a tile: reads first, then the writes and loads;
            // the progressive rebuild (more vector work between a load and
            // its LDS write) keeps sched_interleave's order, which measured
            // 133.3-135.6 us against 138.8-141.7 us for it.
            auto pf4_schedule = [&]() __attribute__((always_inline)) {
                constexpr int kMFt = 2 * C::kFM * C::kFN, kRDt = 2 * (C::kFM + C::kFN);
                constexpr int kWRt = C::kAI + (BITS == 8 ? C::kBI : 2 * C::kBI4);
                constexpr int kLDt = C::kAI + (BITS == 8 ? C::kBI : C::kBI4);
                if constexpr (PROG)
                    sched_interleave<kMFt, kRDt, kWRt, kLDt>();
                else
                    sched_reads_first<kMFt, kRDt, kWRt, kLDt>();
            };
            // steady state: every read, write and load of the pair exists, so
            // the body is one basic block and the interleave pattern applies
            for (; k + 6 <= KTs; k += 2) {
                lread(sA1, sB1, fa1, fb1);
                mfmas(fa0, fb0);
                lstore(S0, 0);
                gload(kb + k + 4, S0);
                pf4_schedule();
                __syncthreads();
                lread(sA0, sB0, fa0, fb0);
                mfmas(fa1, fb1);
                lstore(S1, 1);
                gload(kb + k + 5, S1);
                pf4_schedule();
                __syncthreads();
            }
            // last pairs (KTs even)
            for (; k < KTs; k += 2) {
                lread(sA1, sB1, fa1, fb1);
                mfmas(fa0, fb0);
                if (k + 2 < KTs) lstore(S0, 0);
                if (k + 4 < KTs) gload(kb + k + 4, S0);
                __syncthreads();
                if (k + 2 < KTs) lread(sA0, sB0, fa0, fb0);
                mfmas(fa1, fb1);
                if (k + 3 < KTs) lstore(S1, 1);
                if (k + 5 < KTs) gload(kb + k + 5, S1);
                __syncthreads();
            }
        } else if constexpr (PF == 1) {
            // this block's K tiles kb .. kb + KTs - 1 (a split K range on
            // 128 x 128 tiles; the host keeps each range a whole number of
            // 128-channel groups)
            const int KTs = BM == kSplitTile ? KT / a.ksplit : KT;
            const int kb = BM == kSplitTile ? split * KTs : 0;
            Regs R;
            gload(kb, R);
            lstore(R, 0);
            __syncthreads();
            for (int kt = 0; kt < KTs; ++kt) {
                const int cur = kt & 1;
                if (kt + 1 < KTs) gload(kb + kt + 1, R);
                mma_tile(cur ? sA1 : sA0, cur ? sB1 : sB0);
                if (kt + 1 < KTs) lstore(R, cur ^ 1);
                __syncthreads();
            }
        }
    }

    if (BM == kSplitTile && a.ksplit > 1) {
        // Split K: every block of the tile stores its exact int32 partial
        // tile, then arrives on the tile counter; the last to arrive adds
        // the others' partials and finishes the tile, the others leave.
        // Nobody waits for anybody.  The partials are
        // stored and loaded with device-scope coherent accesses (the sc1
        // bit: what relaxed agent-scope atomics compile to), 16 bytes per
        // lane -- dword-wide coherent loads took 15 us for a 64 KiB
        // partial, these 1.3 us -- and each wave's stores are
        // acknowledged before its block arrives, so the second block
        // reads complete data.  Integer sums: the result does not depend
        // on the arrival order.  (The K-pair kernels arrive here after the
        // barrier that ends their loop, the others after their last one.)
        constexpr int kF = C::kFM * C::kFN;
        constexpr int64_t kSlot = (int64_t)C::kNW * kF * 16 * kWave;  // int32 per partial
        constexpr int kCoherent = 16;  // buffer cache-policy bit sc1 (device scope)
        const int S = a.ksplit;
        // slot layout, 16-byte units: [wave][fragment][e / 4][lane]
        const __amdgpu_buffer_rsrc_t rP =
            make_rsrc(reinterpret_cast<const uint8_t*>(a.part + (int64_t)tbid * S * kSlot),
                      (int64_t)S * kSlot * 4);
        auto unit = [&](int t, int f, int q) {
            return (int)((t * kSlot / 4 + (int64_t)((wave * kF + f) * 4 + q) * kWave + lane) * 16);
        };
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
            for (int j = 0; j < C::kFN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4i v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                   acc[i][j][4 * q + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(v, rP, unit(split, i * C::kFN + j, q), 0,
                                                           kCoherent);
                }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        __shared__ int second;
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(a.sync + tbid, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            second = old == S - 1;
            // every block has arrived: clear the counter for the next call
            if (old == S - 1)
                __hip_atomic_store(a.sync + tbid, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!second) {
            clk_end();
            return;
        }
        for (int t = 0; t < S; ++t) {
            if (t == split) continue;
#pragma unroll
            for (int i = 0; i < C::kFM; ++i)
#pragma unroll
                for (int j = 0; j < C::kFN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4i v = __builtin_amdgcn_raw_buffer_load_b128(
                            rP, unit(t, i * C::kFN + j, q), 0, kCoherent);
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += v[e];
                    }
        }
    }

    // ---- epilogue -------------------------------------------------------------------
    // 32x32 fragment layout: lane l, element e -> row 8*(e/4) + 4*(l/32) + e%4, col l%32.
    // (1) The first round of outlier tiles (up to kRC chunks of 32 columns of
    //     X_out and w_out) starts loading straight into the operand buffers the
    //     K loop has freed -- one load latency, not one per chunk;
    // (2) meanwhile the int32 accumulators are dequantized and scaled in place;
    // (3) per fragment, the f16 outlier MFMAs accumulate onto the scaled tile
    //     (its fp32 values are their C operand: one accumulator set), and in
    //     the last round each finished fragment is stored at once, so that its
    //     stores drain while the next fragment's MFMAs run.
    constexpr int kRC = STAGES == 4 ? 4 : 2;  // outlier chunks per round (one per stage array)
    // chunk c of a round in stage array (c + 2 cf) mod 4: the prefetched
    // chunks 0 and 1 sit in the pair buffer the K loop freed first
    auto stage = [&](int c) __attribute__((always_inline)) -> uint8_t* {
        const int k = (c + 2 * cf) & 3;
        return k == 0 ? sS0 : k == 1 ? sS1 : k == 2 ? sS2 : sS3;
    };
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rXo =
        make_rsrc(reinterpret_cast<const uint8_t*>(a.X_out) + (int64_t)m0 * ldb,
                  nchunks > 0 ? (int64_t)rows_a * ldb : 0);
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t rWo =
        make_rsrc(reinterpret_cast<const uint8_t*>(a.w_out) + (int64_t)n0 * ldb,
                  nchunks > 0 ? (int64_t)rows_b * ldb : 0);
    // chunk c0 + c of both tiles into stage array c, laid out like a 64-byte
    // K tile: row r's 16-byte piece p at slot p ^ swz(r)
    auto load_round = [&](int c0, int nch, int skip) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int c = 0; c < kRC; ++c) {
            if (c >= skip && c < nch) {
                uint8_t* stg = stage(c);
#pragma unroll
                for (int i = 0; i < C::kAI; ++i) {
                    const int row = (i * C::kNW + wave) * 16 + (lane >> 2);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rXo, (lds_ptr_t)(stg + ((i * C::kNW + wave) * 16) * kBK), 16,
                        row * ldb + (((lane & 3) ^ swz(row)) << 4), (c0 + c) * kBK, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < C::kBI; ++i) {
                    const int row = (i * C::kNW + wave) * 16 + (lane >> 2);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rWo, (lds_ptr_t)(stg + BM * kBK + ((i * C::kNW + wave) * 16) * kBK), 16,
                        row * ldb + (((lane & 3) ^ swz(row)) << 4), (c0 + c) * kBK, 0, 0);
                }
            }
        }
#endif
    };
    if (nchunks > 0) load_round(0, min(kRC, nchunks), pre);

    if constexpr (DEBUG) {
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
            for (int j = 0; j < C::kFN; ++j) {
                const int col = n0 + wn * C::kWTN + j * 32 + fr;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + wm * C::kWTM + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                    if (row < a.M && col < a.N)
                        a.acc_debug[(int64_t)row * a.N + col] = acc[i][j][e];
                }
            }
    }
    // dequantize and scale in place: Y_low = (float(acc) * s_x) * s_w
#pragma unroll
    for (int i = 0; i < C::kFM; ++i) {
#pragma unroll
        for (int j = 0; j < C::kFN; ++j) {
            const float swj = sw_t[wn * C::kWTN + j * 32 + fr];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 sx4 = *reinterpret_cast<const float4*>(
                    &sx_t[wm * C::kWTM + i * 32 + 8 * q + 4 * fh]);
                const float sxe[4] = {sx4.x, sx4.y, sx4.z, sx4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][j][4 * q + r] =
                        __float_as_int(((float)acc[i][j][4 * q + r] * sxe[r]) * swj);
            }
            // 256 x 256 tiles: the accumulators fill the 256 AGPRs; left to
            // itself the allocator moves the scaled tile into VGPRs, which
            // do not hold it beside the epilogue's other values, and spills
            // (200-400 bytes per lane, written to HBM).  Keeping each scaled
            // fragment in AGPRs (the outlier MFMAs read and write them there,
            // the stores take them from there) leaves no spill.
            if constexpr (C::kFM * C::kFN * 16 == 256) asm volatile("" : "+a"(acc[i][j]));
        }
    }

    // ---- outlier product: fp16 x fp16 -> fp32, accumulated onto the scaled tile -------
    for (int c0 = 0; c0 < nchunks; c0 += kRC) {
        const int nch = min(kRC, nchunks - c0);
        if (c0 > 0) {
            __syncthreads();  // every wave is done with the previous round's tiles
            load_round(c0, nch, 0);
        }
        MIXQ_WAIT_VMCNT(0);
        __syncthreads();
        // one chunk (32 columns) at a time: its B fragments of every column
        // block and A fragments of every row block in registers, then the
        // MFMAs with the two 16-column steps outermost, so that 16
        // independent accumulations separate the two that share a fragment
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            const uint8_t* stg = stage(c);
            v8h bfr[C::kFN][2], afr[C::kFM][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int j = 0; j < C::kFN; ++j)
                    bfr[j][ks] = *reinterpret_cast<const v8h*>(stg + BM * kBK + rdB[ks] + j * 32 * kBK);
#pragma unroll
                for (int i = 0; i < C::kFM; ++i)
                    afr[i][ks] = *reinterpret_cast<const v8h*>(stg + rdA[ks] + i * 32 * kBK);
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < C::kFM; ++i)
#pragma unroll
                    for (int j = 0; j < C::kFN; ++j)
                        acc[i][j] = __builtin_bit_cast(
                            v16i, __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                      afr[i][ks], bfr[j][ks], __builtin_bit_cast(v16f, acc[i][j]),
                                      0, 0, 0));
        }
    }

    // ---- stores ---------------------------------------------------------------------
    // Offsets are 32-bit and relative to the tile's first row (the host keeps
    // 256 rows of Y below 2^31 bytes); rows past M also fall outside the
    // buffer.  The stores follow the outlier MFMAs in fragment order, so the
    // first fragments' stores issue while the last MFMAs still run.
    const int esz = a.out_mode == MIXQ_OUT_F32 ? 4 : 2;  // bytes per Y element
    const int ldyb = (int)a.ldy * esz;
    const __amdgpu_buffer_rsrc_t rY = make_rsrc(reinterpret_cast<const uint8_t*>(a.Y) +
                                                    (int64_t)m0 * a.ldy * esz,
                                                (int64_t)rows_a * a.ldy * esz);
    if (a.out_mode == MIXQ_OUT_SWIGLU_F16) {
        // A gated weight interleaves 32-row blocks of gate and up rows, and
        // every wave's column range is a multiple of 64, so fragments 2jj and
        // 2jj+1 of a lane hold gate and up of the same (token, output) pairs.
        auto swiglu16 = [&](int32_t gb, int32_t ub) __attribute__((always_inline)) -> uint32_t {
            const float g = __int_as_float(gb);
            const float u = __int_as_float(ub);
            // silu(g) = g / (1 + e^-g), with the hardware reciprocal (1 ulp)
            // in place of an IEEE division: the result is rounded to fp16
            // (2^-11 relative) right after.  g -> -inf: e^-g = inf, rcp = 0.
            const float y = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
            return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)y);
        };
        if (rows_a == BM && n0 + BN <= a.N &&
            ((reinterpret_cast<uintptr_t>(a.Y) | (uintptr_t)ldyb) & 3) == 0) {
            // a whole tile: two outputs per 4-byte store, as the 16-bit
            // output modes below (adjacent lanes swap one value)
            const bool odd = fr & 1;
            const int voff = (4 * fh + (odd ? 1 : 0)) * ldyb +
                             ((n0 + wn * C::kWTN) / 2 + fr - (odd ? 1 : 0)) * 2;
#pragma unroll
            for (int i = 0; i < C::kFM; ++i)
#pragma unroll
                for (int jj = 0; jj < C::kFN / 2; ++jj)
#pragma unroll
                    for (int e = 0; e < 16; e += 2) {
                        const uint32_t h0 = swiglu16(acc[i][2 * jj][e], acc[i][2 * jj + 1][e]);
                        const uint32_t h1 =
                            swiglu16(acc[i][2 * jj][e + 1], acc[i][2 * jj + 1][e + 1]);
                        const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp(
                            (int)(odd ? h0 : h1), 0xB1, 0xF, 0xF, false);
                        const uint32_t w = odd ? (got | (h1 << 16)) : (h0 | (got << 16));
                        __builtin_amdgcn_raw_buffer_store_b32(
                            w, rY, voff + jj * 64,
                            (wm * C::kWTM + i * 32 + 8 * (e >> 2) + (e & 3)) * ldyb, 0);
                    }
            clk_end();
            return;
        }
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::kFN / 2; ++jj) {
                const int pc = n0 + wn * C::kWTN + jj * 64;  // packed column of the gate block
                const int oc = pc / 2 + fr;                   // output column
                const int r0 = wm * C::kWTM + i * 32 + 4 * fh;
                if (pc + fr < a.N) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int rl = r0 + 8 * (e >> 2) + (e & 3);
                        if (rl < rows_a)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                (unsigned short)swiglu16(acc[i][2 * jj][e], acc[i][2 * jj + 1][e]),
                                rY, rl * ldyb + oc * 2, 0, 0);
                    }
                }
            }
        clk_end();
        return;
    }
    if (!ROWS && a.out_mode == MIXQ_OUT_F32 && rows_a == BM && n0 + BN <= a.N) {
        // a whole tile: no per-element test; the lane's column and half in the
        // vector offset, the row (the same for the whole wave) in the scalar one
        const int voff = 4 * fh * ldyb + (n0 + wn * C::kWTN + fr) * 4;
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
            for (int j = 0; j < C::kFN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        acc[i][j][e], rY, voff + j * 128,
                        (wm * C::kWTM + i * 32 + 8 * (e >> 2) + (e & 3)) * ldyb, 0);
        clk_end();
        return;
    }
    const bool bf16 = a.out_mode == MIXQ_OUT_BF16;
    // 16-bit value of an fp32 output: round to nearest, ties to even
    auto to16 = [&](int32_t v) __attribute__((always_inline)) -> uint32_t {
        const float y = __int_as_float(v);
        const uint32_t u = __float_as_uint(y);
        return bf16 ? (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16
                    : (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)y);
    };
    if (!ROWS && esz == 2 && rows_a == BM && n0 + BN <= a.N &&
        ((reinterpret_cast<uintptr_t>(a.Y) | (uintptr_t)ldyb) & 3) == 0) {
        // A whole tile of 16-bit outputs, two per 4-byte store: 2-byte
        // stores (one value per lane) took 15 us longer than the fp32 tile
        // at the prefill shape, half the bytes notwithstanding.  Lanes 2k
        // and 2k+1 hold columns 2k and 2k+1 of the same rows; for each pair
        // of rows (r, r+1) of a fragment the even lane takes its partner's
        // row-r value and stores row r, columns 2k..2k+1, the odd lane takes
        // its partner's row-(r+1) value and stores row r+1 (one DPP swap of
        // adjacent lanes per pair).  Y and its row stride 4-byte aligned.
        const bool odd = fr & 1;
        const int voff = (4 * fh + (odd ? 1 : 0)) * ldyb + (n0 + wn * C::kWTN + fr - (odd ? 1 : 0)) * 2;
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
            for (int j = 0; j < C::kFN; ++j)
#pragma unroll
                for (int e = 0; e < 16; e += 2) {
                    const uint32_t h0 = to16(acc[i][j][e]);      // row r
                    const uint32_t h1 = to16(acc[i][j][e + 1]);  // row r + 1
                    // quad_perm [1, 0, 3, 2]: swap with the adjacent lane
                    const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp(
                        (int)(odd ? h0 : h1), 0xB1, 0xF, 0xF, false);
                    const uint32_t w = odd ? (got | (h1 << 16)) : (h0 | (got << 16));
                    __builtin_amdgcn_raw_buffer_store_b32(
                        w, rY, voff + j * 64,
                        (wm * C::kWTM + i * 32 + 8 * (e >> 2) + (e & 3)) * ldyb, 0);
                }
        clk_end();
        return;
    }
#pragma unroll
    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
        for (int j = 0; j < C::kFN; ++j) {
            const int col = n0 + wn * C::kWTN + j * 32 + fr;
            const int r0 = wm * C::kWTM + i * 32 + 4 * fh;  // tile-relative row of e = 0
            int ycol = col;  // Y column: the packed row, or its W row for a row subset
            if constexpr (ROWS) {
                if (col < a.N) {
                    const int32_t src = a.rmap[col];
                    ycol = (src >= 0 && src < a.n_out) ? src : -1;
                }
            }
            if (col < a.N && (!ROWS || ycol >= 0)) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int rl = r0 + 8 * (e >> 2) + (e & 3);
                    if (rl < rows_a) {
                        if (esz == 4) {
                            __builtin_amdgcn_raw_buffer_store_b32(acc[i][j][e], rY,
                                                                  rl * ldyb + ycol * 4, 0, 0);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b16(
                                (unsigned short)to16(acc[i][j][e]), rY, rl * ldyb + ycol * 2, 0, 0);
                        }
                    }
                }
            }
        }
    clk_end();
}

template <int BM, int BN, int WM, int WN, int BITS, int STAGES, int PF = 1, bool PROG = false,
          bool ROWS = false>
int launch_cfg(GemmArgs a, bool debug, hipStream_t st) {
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = (a.n_end - a.n_begin + BN - 1) / BN;
    const dim3 grid(a.tiles_m * a.tiles_n * a.ksplit), block(WM * WN * kWave);
    if (debug)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, BITS, STAGES, PF, true, PROG, ROWS>), grid,
                           block, 0, st, a);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, BITS, STAGES, PF, false, PROG, ROWS>),
                           grid, block, 0, st, a);
    return launch_status();
}

// Kernel variants (ids of mixq_set_gemm_variant; 0 = automatic choice).
enum {
    kCfgAuto = 0,
    kCfg256x256 = 1,    // 4 waves of 128x128, 64-byte K steps, register-staged (any K)
    kCfg128x128 = 2,    // 4 waves of 64x64, 64-byte K steps, register-staged (any K)
    kCfg256x256SP = 3,  // 4 waves of 128x128, cross-tile software pipeline (INT4 weights)
    kCfg256x256KS = 4,  // 4 waves of 128x128, 128-byte K pairs, issue order pinned (INT8)
    kCfg128x128KP = 5,  // 4 waves of 64x64, 128-byte K pairs (INT8; split K for thin products)
    kCfg128x128SP = 6,  // 4 waves of 64x64, cross-tile software pipeline (INT4 weights)
    kCfgCount = 7,
};

std::atomic<int> g_forced_variant{0};
std::atomic<int64_t*> g_clock_buf{nullptr};
std::atomic<int32_t> g_clock_n{0};

int pick_cfg(int64_t M, int64_t N, int64_t K, int bits) {
    const int f = g_forced_variant.load(std::memory_order_relaxed);
    if (f != kCfgAuto) {
        // a forced variant falls back where its loader does not apply
        if (f >= kCfg256x256SP && K % 128 != 0) return kCfg128x128;
        if (f == kCfg128x128SP && bits == 8) return kCfg128x128KP;
        if (f == kCfg256x256KS && bits == 4) return kCfg256x256SP;
        if (f == kCfg128x128KP && bits == 4) return kCfg128x128;
        return f;
    }
    // Large 256x256 tiles (software-pipelined when K allows) once they give
    // about one tile per CU; 128x128 tiles (K pairs for INT8 weights) for
    // thinner products.
    const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
    if (big >= 192) {
        if (K % 128 != 0) return kCfg256x256;
        return bits == 8 ? kCfg256x256KS : kCfg256x256SP;
    }
    return bits == 8 && K % 128 == 0 ? kCfg128x128KP : kCfg128x128;
}

template <bool ROWS = false>
int launch_w8(const GemmArgs& a, int cfg, bool debug, hipStream_t st) {
    switch (cfg) {
        case kCfg256x256KS: return launch_cfg<256, 256, 2, 2, 8, 4, 6, false, ROWS>(a, debug, st);
        case kCfg128x128KP: return launch_cfg<128, 128, 2, 2, 8, 4, 5, false, ROWS>(a, debug, st);
        case kCfg256x256:
            if constexpr (!ROWS) return launch_cfg<256, 256, 2, 2, 8, 2>(a, debug, st);
            [[fallthrough]];
        default: return launch_cfg<128, 128, 2, 2, 8, 2, 1, false, ROWS>(a, debug, st);
    }
}

template <bool PROG, bool ROWS = false>
int launch_w4_t(const GemmArgs& a, int cfg, bool debug, hipStream_t st) {
    switch (cfg) {
        case kCfg256x256: return launch_cfg<256, 256, 2, 2, 4, 2, 1, PROG, ROWS>(a, debug, st);
        case kCfg256x256SP: return launch_cfg<256, 256, 2, 2, 4, 2, 4, PROG, ROWS>(a, debug, st);
        case kCfg128x128SP: return launch_cfg<128, 128, 2, 2, 4, 2, 4, PROG, ROWS>(a, debug, st);
        default: return launch_cfg<128, 128, 2, 2, 4, 2, 1, PROG, ROWS>(a, debug, st);
    }
}

int launch_w4(const GemmArgs& a, int cfg, bool debug, hipStream_t st) {
    if (a.rmap) return launch_w4_t<true, true>(a, cfg, debug, st);  // progressive rows only
    return a.gsz ? launch_w4_t<true>(a, cfg, debug, st) : launch_w4_t<false>(a, cfg, debug, st);
}

int launch_bits(const GemmArgs& a, int cfg, bool debug, hipStream_t st) {
    if (a.wbits == 8)
        return a.rmap ? launch_w8<true>(a, cfg, debug, st) : launch_w8(a, cfg, debug, st);
    return launch_w4(a, cfg, debug, st);
}

}  // namespace
}  // namespace mixq

namespace mixq {
namespace {

// ---- the GEMM with the library's own split-K workspace -----------------------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops): the split-K workspace of mixq_gemm_ex lives in a
// file-scope device array instead of caller memory.  Each device that runs
// the library holds its own copy for the life of the process; its address
// is taken once per device with hipGetSymbolAddress (the array's name is
// only a host-side handle) and kept.  The tile counters at its start must
// be zero before a call; every completed call leaves them zero, and the
// first call on a device clears them with a fill kernel on its stream.

// every plan on 256 CUs fits: at most two 128 x 128 partial tiles per compute unit
constexpr size_t kScratchBytes = (size_t)kSplitSyncBytes + 512 * (size_t)kSplitSlotBytes;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void clear_words_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Device address of this device's scratch array (cleared on first use), or
// null on a HIP error.
void* scratch_ptr(hipStream_t st) {
    static std::mutex mu;
    static void* ptr[64];
    static bool ready[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ready[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        hipLaunchKernelGGL(clear_words_kernel, dim3(4), dim3(256), 0, st, static_cast<uint32_t*>(p),
                           (int)(kSplitSyncBytes / 4));
        if (hipGetLastError() != hipSuccess) return nullptr;
        ptr[dev] = p;
        ready[dev] = true;
    }
    return ptr[dev];
}


int gemm_impl(const int8_t* Xq, const float* s_x, const uint16_t* X_out,
              const mixq_act_state* state, const mixq_weight* w, int64_t M, float* Y,
              int64_t ldy, int32_t* acc_debug, void* ws, size_t ws_bytes, void* stream,
              int32_t out_mode = MIXQ_OUT_F32, bool own_ws = false) {
    if (!Xq || !s_x || !state || !w || !Y) return MIXQ_ERR_INVALID_ARG;
    if (!state->count || !w->wq || !w->s_w) return MIXQ_ERR_INVALID_ARG;
    if (out_mode != MIXQ_OUT_F32 && out_mode != MIXQ_OUT_SWIGLU_F16 && out_mode != MIXQ_OUT_F16 &&
        out_mode != MIXQ_OUT_BF16)
        return MIXQ_ERR_INVALID_ARG;
    if (out_mode == MIXQ_OUT_SWIGLU_F16 && (w->gated != 1 || w->N % 64 != 0))
        return MIXQ_ERR_INVALID_ARG;
    if (w->group != 0 && (w->group != MIXQ_PROGRESSIVE_GROUP || w->bits != 4 || !w->gsz))
        return MIXQ_ERR_INVALID_ARG;
    if (w->group != 0 && w->K % MIXQ_PROGRESSIVE_GROUP != 0) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    // the group table's byte offsets are 32-bit
    if (w->group != 0 && w->N * (w->K / MIXQ_PROGRESSIVE_GROUP) * 2 > 0x7FFFFFFF)
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    // row subsets: INT8 or progressive INT4 rows, fp32 output
    if (w->rmap && (w->gated || out_mode != MIXQ_OUT_F32 || w->n_out < 1 ||
                    (w->bits == 4 && w->group == 0)))
        return MIXQ_ERR_INVALID_ARG;
    // Y columns: N, N / 2 for SwiGLU, n_out for a row subset
    const int64_t ny = w->rmap ? w->n_out : out_mode == MIXQ_OUT_SWIGLU_F16 ? w->N / 2 : w->N;
    if (M <= 0 || w->N <= 0 || w->K <= 0 || ldy < ny) return MIXQ_ERR_INVALID_ARG;
    if (w->bits != 8 && w->bits != 4) return MIXQ_ERR_INVALID_ARG;
    if (state->k_cap < 0 || state->k_cap > w->K || w->k_cap != state->k_cap)
        return MIXQ_ERR_INVALID_ARG;
    if (state->k_cap > 0 && (!X_out || !w->w_out)) return MIXQ_ERR_INVALID_ARG;
    if (!valid_k(w->K)) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (M > (1 << 30) || w->N > (1 << 30)) return MIXQ_ERR_UNSUPPORTED_SHAPE;
    // Y stores use 32-bit byte offsets from the tile's first row (256 rows at
    // most); the grid is one dimension (128 x 128 tiles, K split up to 4 ways)
    if (ldy * (out_mode == MIXQ_OUT_F32 ? 4 : 2) * 256 > (int64_t)0x7FFFFFFF)
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (((M + 127) / 128) * ((w->N + 127) / 128) * 4 > (int64_t)0x7FFFFFFF)
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    if (((uintptr_t)Xq & 15u) || ((uintptr_t)w->wq & 15u) || ((uintptr_t)X_out & 15u) ||
        ((uintptr_t)w->w_out & 15u) || ((uintptr_t)ws & 15u))
        return MIXQ_ERR_UNSUPPORTED_SHAPE;
    int rc = check_device_cached();
    if (rc != MIXQ_OK) return rc;

    GemmArgs a;
    a.Xq = Xq;
    a.s_x = s_x;
    a.X_out = X_out;
    a.count = state->count;
    a.wq = w->wq;
    a.s_w = w->s_w;
    a.w_out = w->w_out;
    a.ld_out = (int32_t)outlier_ld(state->k_cap);
    a.M = (int32_t)M;
    a.N = (int32_t)w->N;
    a.K = (int32_t)w->K;
    a.Y = Y;
    a.ldy = ldy;
    a.acc_debug = acc_debug;
    a.tiles_m = a.tiles_n = 0;
    a.n_begin = 0;
    a.n_end = a.N;
    a.wbits = w->bits;
    a.clk = g_clock_buf.load(std::memory_order_relaxed);
    a.clk_n = a.clk ? g_clock_n.load(std::memory_order_relaxed) : 0;
    a.ksplit = 1;
    a.sync = nullptr;
    a.part = nullptr;
    a.out_mode = out_mode;
    a.gsz = w->group ? w->gsz : nullptr;
    a.rmap = w->rmap;
    a.n_out = w->rmap ? w->n_out : 0;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    const int f = g_forced_variant.load(std::memory_order_relaxed);
    const int pc = pick_cfg(M, w->N, w->K, w->bits);
    if (own_ws) {
        // the library's scratch array stands in for ws, set up only when the
        // plan below splits K (the same conditions)
        ws = nullptr;
        ws_bytes = 0;
        int St0 = 1;
        const bool split = (f == kCfgAuto || f == kCfg128x128KP) && pc == kCfg128x128KP &&
                           split_plan(M, w->N, w->K, w->bits, device_cu_count()) > 1;
        const bool tail = f == kCfgAuto && (pc == kCfg256x256KS || pc == kCfg256x256SP) &&
                          tail_plan(M, w->N, w->K, device_cu_count(), &St0) > 0 && St0 > 1;
        if (split || tail) {
            ws = scratch_ptr(st);
            if (!ws) return MIXQ_ERR_HIP;
            ws_bytes = kScratchBytes;
        }
    }
    const int S = ws && (f == kCfgAuto || f == kCfg128x128KP) && pc == kCfg128x128KP
                      ? split_plan(M, w->N, w->K, w->bits, device_cu_count())
                      : 1;
    if (S > 1 && (int64_t)ws_bytes < split_workspace_bytes(M, w->N, S)) return MIXQ_ERR_WORKSPACE;
    if (S > 1) {
        a.ksplit = S;
        a.sync = static_cast<int32_t*>(ws);
        a.part = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + kSplitSyncBytes);
        return a.rmap ? launch_cfg<128, 128, 2, 2, 8, 4, 5, false, true>(a, acc_debug != nullptr, st)
                      : launch_cfg<128, 128, 2, 2, 8, 4, 5>(a, acc_debug != nullptr, st);
    }
    const bool dbg = acc_debug != nullptr;
    // Tail split: when the 256 x 256 tiles come to one round of the device
    // plus a short second round (N a little above a multiple of the columns
    // one round holds), the second round would cost a whole tile time for a
    // few tiles.  Instead the 256 x 256 launch takes the tile columns that
    // fill one round, and a second launch covers the remaining columns with
    // 128 x 128 tiles, four times as many blocks, each a quarter of the work.
    // With a workspace the tail's K is split as well, so that its blocks
    // fill the device (tail_plan).
    int St = 1;
    const int n_split = f == kCfgAuto && (pc == kCfg256x256KS || pc == kCfg256x256SP)
                            ? tail_plan(M, w->N, w->K, device_cu_count(), &St)
                            : 0;
    if (n_split > 0) {
        const int tail_cfg = w->bits == 8 ? kCfg128x128KP : kCfg128x128SP;
        GemmArgs a2 = a;
        a.n_end = n_split;
        a2.n_begin = n_split;
        if (St > 1 && ws && (int64_t)ws_bytes < tail_workspace_bytes(M, w->N, n_split, St))
            return MIXQ_ERR_WORKSPACE;
        if (St > 1 && ws) {
            a2.ksplit = St;
            a2.sync = static_cast<int32_t*>(ws);
            a2.part = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + kSplitSyncBytes);
        }
        rc = launch_bits(a, pc, dbg, st);
        if (rc != MIXQ_OK) return rc;
        return launch_bits(a2, tail_cfg, dbg, st);
    }
    return launch_bits(a, pc, dbg, st);
}

}  // namespace
}  // namespace mixq

extern "C" int mixq_set_clock_record(int64_t* buf, int32_t n_blocks) {
    if ((buf == nullptr) != (n_blocks == 0) || n_blocks < 0) return MIXQ_ERR_INVALID_ARG;
    mixq::g_clock_n.store(n_blocks, std::memory_order_relaxed);
    mixq::g_clock_buf.store(buf, std::memory_order_relaxed);
    return MIXQ_OK;
}

extern "C" int mixq_set_gemm_variant(int32_t variant) {
    if (variant < 0 || variant >= mixq::kCfgCount) return MIXQ_ERR_INVALID_ARG;
    mixq::g_forced_variant.store(variant, std::memory_order_relaxed);
    return MIXQ_OK;
}

extern "C" int mixq_gemm(const int8_t* Xq, const float* s_x, const uint16_t* X_out,
                         const mixq_act_state* state, const mixq_weight* w, int64_t M, float* Y,
                         int64_t ldy, int32_t* acc_debug, void* stream) {
    return mixq::gemm_impl(Xq, s_x, X_out, state, w, M, Y, ldy, acc_debug, nullptr, 0, stream);
}

extern "C" int mixq_gemm_ws(const int8_t* Xq, const float* s_x, const uint16_t* X_out,
                            const mixq_act_state* state, const mixq_weight* w, int64_t M,
                            float* Y, int64_t ldy, int32_t* acc_debug, void* ws, size_t ws_bytes,
                            void* stream) {
    return mixq::gemm_impl(Xq, s_x, X_out, state, w, M, Y, ldy, acc_debug, ws, ws_bytes, stream);
}

extern "C" int mixq_gemm_ex(const int8_t* Xq, const float* s_x, const uint16_t* X_out,
                            const mixq_act_state* state, const mixq_weight* w, int64_t M, void* Y,
                            int64_t ldy, int32_t out_mode, int32_t* acc_debug, void* ws,
                            size_t ws_bytes, void* stream) {
    return mixq::gemm_impl(Xq, s_x, X_out, state, w, M, static_cast<float*>(Y), ldy, acc_debug,
                           ws, ws_bytes, stream, out_mode);
}

extern "C" size_t mixq_gemm_scratch_bytes(void) { return mixq::kScratchBytes; }

extern "C" int mixq_gemm_noalloc(const int8_t* Xq, const float* s_x, const uint16_t* X_out,
                                 const mixq_act_state* state, const mixq_weight* w, int64_t M,
                                 void* Y, int64_t ldy, int32_t out_mode, int32_t* acc_debug,
                                 void* stream) {
    return mixq::gemm_impl(Xq, s_x, X_out, state, w, M, static_cast<float*>(Y), ldy, acc_debug,
                           nullptr, 0, stream, out_mode, /*own_ws=*/true);
}
