// bf16 relu(A·B) on the gfx950 matrix cores, "ping-pong" schedule: eight
// wave64s per output tile (256 x 256, or 128 x 256), two on each SIMD, split
// into two groups of four. Between two consecutive barriers one group only
// runs MFMAs while the other only reads operand fragments from LDS and issues
// global->LDS copies; at the barrier the roles swap. Each SIMD therefore
// always has one wave feeding its matrix core and one wave doing memory work,
// and the hardware issues both streams side by side.
//
// The arithmetic is the lecture's tiled matmul with the fused activation
// ("Kernels, Triton, XLA", section "Reductions and tiling", and the Chinese
// notes' section 5.5): per output tile, K is swept in slabs staged in LDS,
// fp32 accumulation (v_mfma_f32_16x16x32_bf16), the fused epilogue on the
// accumulator (optional per-column bias, then ReLU by default, or GeLU's
// tanh form, or nothing), one rounding to bf16 (nearest, ties to even), one
// masked store.
//
// Waves: wave w belongs to group w / 4; within a group, (wm, wn') =
// ((w%4)/2, (w%4)%2) and the wave owns rows (BM/2)*wm .. +BM/2 and columns
// 64*(wn' + 2*group) .. +64 of the tile (BM/32 x 4 MFMA blocks; 128 fp32
// accumulators per lane for the 256-row tile). Slabs are 32 deep along K and
// every interval between two barriers covers a PAIR of slabs, 64 k.
//
// LDS: A is staged per pair of slabs (64 k, 128 bytes per row) in a ring of
// three stages (BM x 128 bytes each), B per slab in a ring of four 16 KB
// stages (160 KB in all for the 256-row tile).
//  - A stage: row r's 16-byte chunk c sits at r*128 + 16*(c ^ (r%8)). One
//    copy instruction moves 8 rows x 128 bytes: lane 8r'+j fetches chunk
//    j ^ r' of its row, so each group of 8 lanes reads one whole 128-byte
//    line from global memory and writes it, permuted, to one LDS row. A
//    fragment reads (16 lanes: 16 rows, one chunk) hit 16 distinct chunk
//    positions and run at the full LDS rate.
//  - B stage: 32 rows of 512 bytes, 16-byte chunks XOR-swizzled by row, read
//    with ds_read_b64_tr_b16 (each lane gets 8 consecutive k of a column).
// Group 1 copies A, group 0 copies B; per interval every wave of group 0
// issues eight 1 KB copies (two B slabs), every wave of group 1 BM/32 (the
// A pair).
//
// Why 64-deep intervals: a memory interval's fragment reads take longer than
// 32 MFMAs (about 640 cycles against 512, measured on a register-and-LDS
// probe), so one slab per interval would leave the matrix cores idle at
// every barrier; 64 MFMAs cover the reads of two slabs, and the barriers
// halve. The memory role holds both slabs' fragments in two register sets.
//
// Schedule (J_t ends at a barrier; pair p = slabs 2p, 2p+1):
//   prologue: group 1 copies A pairs 0 and 1, group 0 B pair 0; wait for
//             pair 0; barrier. J_-1: group 0 reads pair 0, copies B pair 1.
//   J_2p:   group 0 multiplies pair p, then waits for all its copies (B
//           pair p+1, issued in J_2p-1);
//           group 1 reads pair p, copies A pair p+2, then waits for all but
//           those (A pair p+1, issued in J_2p-2).
//   J_2p+1: group 0 reads pair p+1 and copies B pair p+2 (into the stages
//           of pair p, which group 1 read in J_2p);
//           group 1 multiplies pair p.
// A pair p+2's stage last held pair p-1, read by group 1 in J_2p-2.
// Copies are issued only for pairs that hold some k < K (the prologue's
// copies of pair 1 aside); the last pairs are peeled off both loops, so the
// loops themselves have no branches.
// End of the tile: group 0's last MFMAs come one interval before group 1's,
// and group 0 stores its half of the tile in that interval, while group 1
// runs the tile's last MFMAs; group 1 stores after the last barrier.
//
// Requires lda, ldb, ldc, K and N to be multiples of 8 and 16-byte aligned
// pointers.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kBN = 256, kBK = 32;
constexpr int kThreads = 512;
constexpr int kNB = 4;                                // MFMA column blocks per wave (64 columns)
constexpr int kStagesA = 3, kStagesB = 4;
constexpr int kStageBBytes = kBK * kBN * 2;           // one slab of B: 16 KB
constexpr int kCopiesB = 4;                           // 1 KB B copies per wave per memory interval

// BM = 256 or 128 tile rows; each wave owns BM/2 x 64 outputs (kMB x 4 MFMA
// blocks). The 128-row tile doubles the tile count for products whose
// 256 x 256 grid leaves CUs idle.
template <int BM>
struct PingPong {
    static_assert(BM == 256 || BM == 128, "tile rows");
    static constexpr int kMB = BM / 32;
    static constexpr int kStageABytes = BM * 2 * kBK * 2;    // one pair of slabs of A (BM x 64 k)
    static constexpr int kBBase = kStagesA * kStageABytes;   // byte offset of the B ring
    static constexpr int kLdsBytes = kBBase + kStagesB * kStageBBytes;
    static constexpr int kCopiesA = BM / 64;                 // 1 KB A copies per wave per memory interval
    static constexpr int kCopies = kCopiesA > kCopiesB ? kCopiesA : kCopiesB;
};

__device__ inline int swz_b(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

template <int BM>
__global__ __launch_bounds__(kThreads, 1) void mmrelu_bf16_pingpong(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C,
    int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m,
    const uint16_t *__restrict__ bias, int act)
{
    using P = PingPong<BM>;
    constexpr int kMB = P::kMB, kStageABytes = P::kStageABytes, kBBase = P::kBBase, kCopies = P::kCopies;
    constexpr int kHalf = BM / 2;                      // rows per half of an A pair, and per wave
    static_assert(P::kLdsBytes <= 160 * 1024, "LDS budget");
    static_assert(kNB == kCopies, "one copy per fragment part");
    __shared__ __attribute__((aligned(1024))) uint16_t lds[P::kLdsBytes / 2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2, wl = wave & 3;
    const int wm = wl >> 1, wn = (wl & 1) + 2 * grp;
    const int g = lane >> 4, t = lane & 15;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * kBN;
    const uint32_t lds0 = lds_address(lds);

    // Copy plans. Group 1, A: copy q (q < BM/64) of half hh of a pair covers
    // rows (BM/2)hh + 8(4q + wl) .. +8; lane 8r'+j fetches chunk c = j ^ r' (8 k) of
    // row r'. Rows past M get an out-of-range offset here, chunks past K per
    // pair. Group 0, B: copy q covers B rows 2(4q + wl) .. +2 of a slab,
    // lane l chunk (l%32) ^ swz(row); columns past N are masked here, rows
    // past K fall outside the B resource rebased to the slab.
    const rsrc_t ra = make_rsrc(A + static_cast<int64_t>(m0) * lda, ((static_cast<int64_t>(M) - 1 - m0) * lda + K) * 2);
    const int a_chunk = (lane & 7) ^ (lane >> 3);
    // (Two separate arrays, selected with ?: below: one array indexed by a
    // run-time half would be placed in scratch memory.)
    uint32_t voff0[kCopies], voff1[kCopies];
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
        if (grp == 1) {
            const int row = 8 * (4 * q + wl) + (lane >> 3);
            voff0[q] = (m0 + row < M) ? static_cast<uint32_t>((row * lda + 8 * a_chunk) * 2) : kOutOfRange;
            voff1[q] = (m0 + kHalf + row < M) ? static_cast<uint32_t>(((row + kHalf) * lda + 8 * a_chunk) * 2)
                                              : kOutOfRange;
        } else {
            const int row = 2 * (4 * q + wl) + (lane >> 5);
            const int col = ((lane & 31) ^ swz_b(row)) * 8;
            voff0[q] = (n0 + col < N) ? static_cast<uint32_t>((row * ldb + col) * 2) : kOutOfRange;
            voff1[q] = kOutOfRange;
        }
    }
    // Copy q (< 8) of A pair p (group 1): half q / kCopiesA, copy q % kCopiesA
    // of that half; the 128-row tile has four copies per pair (q >= 4 issues
    // nothing).
    auto copy_a = [&](int p, int q) __attribute__((always_inline)) {
        if (q >= 2 * P::kCopiesA) return;
        const int hh = q / P::kCopiesA, qq = q % P::kCopiesA;
        const int k0 = 2 * kBK * p;
        const uint32_t off = (8 * a_chunk < K - k0) ? (hh ? voff1[qq] : voff0[qq]) : kOutOfRange;
        const uint32_t st = lds0 + (p % kStagesA) * kStageABytes + (kHalf * hh + 8 * (4 * qq + wl)) * 128;
        load_to_lds<16>(ra, st, off, static_cast<uint32_t>(k0) * 2);
    };
    // Copy q of B slab m (group 0); rb is the B resource rebased to the slab.
    auto b_rsrc = [&](int m) __attribute__((always_inline)) {
        const int k0 = m * kBK;
        return make_rsrc(B + static_cast<int64_t>(k0) * ldb + n0, ((static_cast<int64_t>(K) - 1 - k0) * ldb + N - n0) * 2);
    };
    auto copy_b = [&](int m, int q, const rsrc_t &rb) __attribute__((always_inline)) {
        const uint32_t st = lds0 + kBBase + (m % kStagesB) * kStageBBytes + (4 * q + wl) * 1024;
        load_to_lds<16>(rb, st, voff0[q]);
    };

    // Fragment read plan (element offsets). A block i of slab s: rows
    // wm*BM/2 + 16i + t, chunk 4(s%2) + g of the pair. B block j: columns
    // wn*64 + 16j + 4(t%4), rows 8g + t/4 (+4h) of the slab.
    const int a_off0 = (wm * kHalf + t) * 64 + ((g ^ (t & 7)) << 3);
    const int a_off1 = (wm * kHalf + t) * 64 + (((4 + g) ^ (t & 7)) << 3);
    int b_off[kNB];
    {
        const int k_lane = 8 * g + (t >> 2);
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int n = wn * 64 + j * 16 + 4 * (t & 3);
            b_off[j] = kBBase / 2 + k_lane * kBN + (((n >> 3) ^ swz_b(k_lane)) << 3) + (n & 7);
        }
    }

    // Part p of the fragments of slab s, into register set d (slab s%2 of a
    // pair): B block p (two transposed reads) and A blocks p kMB/4 ..
    // (p+1) kMB/4 - 1 (two, or one for 128 rows).
    bf16x8 fa[2][kMB], fb[2][kNB];
    auto read_part = [&](int s, int p, int d) __attribute__((always_inline)) {
        const uint16_t *sa = lds + ((s >> 1) % kStagesA) * (kStageABytes / 2) + ((s & 1) ? a_off1 : a_off0);
        const uint16_t *sb = lds + (s % kStagesB) * (kStageBBytes / 2);
        i16x4 half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MMRELU_LDS i16x4 *)(sb + b_off[p] + 4 * h * kBN));
        fb[d][p] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int i = p * kMB / kNB; i < (p + 1) * kMB / kNB; ++i)
            fa[d][i] = *reinterpret_cast<const bf16x8 *>(sa + i * 16 * 64);
    };
    // The memory role of one interval: read both slabs of pair pp (if
    // `do_read`) and issue this wave's eight copies, copy(q) before part q
    // (issuing all reads first left the texture unit idle while the LDS
    // worked, and the other way round). The wave raises its issue priority
    // meanwhile, so that its reads and copies go out ahead of the MFMA wave
    // on the same SIMD, whose matrix core has queued work anyway (8192^3:
    // 747 against 754 us; priority 3 gives 749, and raising the MFMA wave
    // instead is slower). Copies are volatile asm with a memory clobber, so
    // the order is kept.
    auto mem_work_pair = [&](int pp, bool do_read, auto &&copy) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int q = 0; q < 2 * kNB; ++q) {
            copy(q);
            if (do_read) read_part(2 * pp + q / kNB, q % kNB, q / kNB);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    f32x4 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfmas = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < 2; ++d)
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int j = 0; j < kNB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[d][j], fa[d][i], acc[i][j], 0, 0, 0);
    };
    // End of an interval: wait until at most `in_flight` of this wave's
    // copies are outstanding (if in_flight >= 0), then the barrier. The
    // fences keep each interval's work between its barriers (MFMAs touch no
    // memory and would otherwise be moved across).
    auto interval_end = [&](int in_flight) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if (in_flight == 8) wait_vmcnt<8>();
        if (in_flight == 4) wait_vmcnt<4>();
        if (in_flight == 0) wait_vmcnt<0>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    // Epilogue: lane (g, t) of block (i, j) holds C[row][col .. col+3]; bias
    // and activation on fp32, round to bf16, one 8-byte masked store. The
    // bias values of the lane's columns are loaded once, up front, and only
    // when there is a bias; stores go row block by row block, so the four
    // column blocks of a row complete its lines back to back.
    auto epilogue = [&]() __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rc = make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0,
                                                          ((static_cast<int64_t>(M) - 1 - m0) * ldc + N - n0) * 2);
        float bj[kNB][4];
        if (bias != nullptr) {
            const __amdgpu_buffer_rsrc_t rb = make_bias_rsrc(bias, n0, N, 2);
#pragma unroll
            for (int j = 0; j < kNB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) bj[j][r] = bias_bf16(rb, wn * 64 + j * 16 + 4 * g + r);
        } else {
#pragma unroll
            for (int j = 0; j < kNB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) bj[j][r] = 0.0f;
        }
        with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
            constexpr int ACT = decltype(act_c)::value;
#pragma unroll
            for (int i = 0; i < kMB; ++i) {
                const int row = wm * kHalf + i * 16 + t;
#pragma unroll
                for (int j = 0; j < kNB; ++j) {
                    const int col = wn * 64 + j * 16 + 4 * g;
                    const f32x4 v = acc[i][j];
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(activate<ACT>(v[r] + bj[j][r]));
                    const uint32_t off =
                        (m0 + row < M && n0 + col < N) ? static_cast<uint32_t>((row * ldc + col) * 2) : kOutOfRange;
                    store_b64(rc, off, __builtin_bit_cast(u32x2, o));
                }
            }
        });
    };
    auto no_copy = [](int) {};

    // Each group runs its own loop (one copy of the fragment registers and
    // the MFMA chain per code path); both execute the same barriers. Copies
    // are issued only for pairs that hold some k < K; the prologue's copies
    // of pair 1 are the exception (masked zero fills when K <= 64).
    const int np = (K + 2 * kBK - 1) / (2 * kBK);
    if (np > 0) {
        if (grp == 1) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int q = 0; q < 2 * kNB; ++q) copy_a(p, q);
        } else {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const rsrc_t rb = b_rsrc(m);
#pragma unroll
                for (int q = 0; q < kCopiesB; ++q) copy_b(m, q, rb);
            }
        }
        interval_end(grp == 1 ? 2 * P::kCopiesA : 0);   // pair 0 has landed
        if (grp == 0) {
            {
                const rsrc_t rb0 = b_rsrc(2), rb1 = b_rsrc(3);
                mem_work_pair(0, true, [&](int q) __attribute__((always_inline)) {
                    copy_b(2 + q / kCopiesB, q % kCopiesB, q < kCopiesB ? rb0 : rb1);
                });                                               // J_-1
            }
            interval_end(-1);
            // J_2p+1 reads pair p+1 and copies B pair p+2 while they exist;
            // the last two pairs are peeled off the loop, so the loop has no
            // branch and the fragment registers are dead by the epilogue.
            int p = 0;
            for (; p + 2 < np; ++p) {
                mfmas();                                          // J_2p
                interval_end(0);                                  // B pair p+1 has landed
                const rsrc_t rb0 = b_rsrc(2 * p + 4), rb1 = b_rsrc(2 * p + 5);
                mem_work_pair(p + 1, true, [&](int q) __attribute__((always_inline)) {
                    copy_b(2 * p + 4 + q / kCopiesB, q % kCopiesB, q < kCopiesB ? rb0 : rb1);
                });                                               // J_2p+1
                interval_end(-1);
            }
            if (p + 1 < np) {                                     // pair np-2: read the last pair
                mfmas();
                interval_end(0);
                mem_work_pair(p + 1, true, no_copy);
                interval_end(-1);
            }
            // The last pair. Nothing is left to read: this group stores its
            // half of the tile while group 1 runs the tile's last MFMAs.
            mfmas();
            interval_end(0);
            epilogue();
            interval_end(-1);
        } else {
            interval_end(-1);                                     // J_-1
            // J_2p reads pair p, copies A pair p+2 while it exists, then waits
            // for pair p+1 (all but the copies just issued, or all).
            int p = 0;
            for (; p + 2 < np; ++p) {
                mem_work_pair(p, true, [&](int q) __attribute__((always_inline)) { copy_a(p + 2, q); });
                interval_end(2 * P::kCopiesA);
                mfmas();                                          // J_2p+1
                interval_end(-1);
            }
            for (; p < np; ++p) {
                mem_work_pair(p, true, no_copy);
                interval_end(0);
                mfmas();
                interval_end(-1);
            }
        }
    }
    if (grp == 1 || np == 0) epilogue();
}

// Tile-row bands of this height are walked column by column inside each XCD's
// range of tiles (tile_of); 4 and 8 tie at 8192^3, 2, 16 and 32 are slower.
constexpr int kGroupM = 8;

template <int BM>
hipError_t launch_pingpong(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + kBN - 1) / kBN;
    hipLaunchKernelGGL((mmrelu_bf16_pingpong<BM>), dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t *>(p.A), static_cast<const uint16_t *>(p.B),
                       static_cast<uint16_t *>(p.C), p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, kGroupM,
                       static_cast<const uint16_t *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

// 256 x 256 tiles: the planner's bf16 tile kernel for large aligned products
// (8192^3: 753 us against 804 for a schedule with one slab per interval).
const Variant *variant_bf16_pingpong256()
{
    static const Variant v = {"mmrelu_bf16_pingpong<256,256,64,A3B4>", MMRELU_DTYPE_BF16, 256, 256, 64, 512, 1, 8,
                              launch_pingpong<256>};
    return &v;
}
// 128 x 256 tiles: twice the tiles of the 256 x 256 grid, for products that
// would leave CUs idle on it. Relative cost per output 1.33: one 128 x 256
// tile of K = 8192 per CU takes 126 us (1024 x 8192 x 8192), a 256 x 256 tile
// 188 us (a quarter of 8192^3).
const Variant *variant_bf16_pingpong128()
{
    static const Variant v = {"mmrelu_bf16_pingpong<128,256,64,A3B4>", MMRELU_DTYPE_BF16, 128, 256, 64, 512, 1, 8,
                              launch_pingpong<128>, 1.33f};
    return &v;
}

}  // namespace mmrelu
