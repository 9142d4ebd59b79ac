// bf16 act(A·B + bias) on the matrix cores for any layout: leading
// dimensions, N and K need not be multiples of 8 nor rows 16-byte aligned,
// which the DMA-fed bf16 kernels require. The lecture's tiled recipe
// ("Kernels, Triton, XLA", section "Reductions and tiling"): one workgroup per
// output tile, K swept in slabs staged in LDS, masked loads that read zeros
// past the edges, fp32 accumulation, the activation on the accumulator, one
// masked store.
//  * BT x BT output tile (BT = 64 or 128) per workgroup of four waves
//    (2 x 2), each wave a BT/2 x BT/2 sub-tile as blocks of
//    v_mfma_f32_16x16x32_bf16; K in slabs of 32.
//  * Operands arrive in 16-byte pieces even when rows are misaligned: the 8
//    elements a lane needs start e elements into an aligned 16-byte chunk,
//    so the lane loads that chunk and the next and shifts the pair by e
//    elements (v_alignbyte). Both loads are aligned and coalesced across the
//    wave; elements past K (A) or past N (B) are then zeroed. Loads go
//    through buffer resources whose range ends at the operand's last 16-byte
//    granule: chunks past it read as zeros, and a 16-byte granule never
//    crosses a page, so the bytes read around the operand are never
//    unmapped.
//  * A chunks land in LDS chunk-major per 16-row block and B rows row-major
//    with XOR-swizzled chunks, the layouts of the aligned kernels, so
//    fragments are one ds_read_b128 (A) and two ds_read_b64_tr_b16 (B).
//  * One slab is loaded into registers while the previous one is
//    multiplied; double-buffered LDS; bias, activation and one rounding to
//    bf16 in the epilogue, which stages the tile in LDS and stores whole
//    rows with the widest stores each row's alignment allows.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kAnyBK = 32, kAnyThreads = 256;

// XOR applied to the 16-byte chunk index of B row k in LDS (BT/8 chunks per
// row): the 16 lanes of a transposed read touch rows k .. k+3 and spread
// over the banks.
template <int BT>
__device__ inline int swz_row(int k)
{
    if constexpr (BT >= 128) return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
    else return (k & 3) << 1;
}

// (a & m) | (b & ~m): a per-lane select written as bit operations, so it
// stays a v_bfi_b32 instead of becoming a branch.
__device__ inline uint32_t pick(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

// The 8 bf16 that start e elements (0 <= e < 8) into the 32 bytes lo:hi, in
// three branch-free steps: shift by two dwords if e & 4, by one dword if
// e & 2, then by half a dword if e & 1 (v_alignbyte).
__device__ inline u32x4 realign(const u32x4 &lo, const u32x4 &hi, int e)
{
    const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const uint32_t m2 = 0u - ((static_cast<uint32_t>(e) >> 2) & 1u);
    const uint32_t m1 = 0u - ((static_cast<uint32_t>(e) >> 1) & 1u);
    const uint32_t sh = (static_cast<uint32_t>(e) & 1u) * 2u;
    uint32_t x[6], y[5];
#pragma unroll
    for (int j = 0; j < 6; ++j) x[j] = pick(m2, w[j + 2], w[j]);
#pragma unroll
    for (int j = 0; j < 5; ++j) y[j] = pick(m1, x[j + 1], x[j]);
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __builtin_amdgcn_alignbyte(y[i + 1], y[i], sh);   // low dword of ({hi, lo} >> 8 sh)
    return out;
}

// Keep the first v of the 8 bf16 in x (v <= 0: none), zero the rest.
__device__ inline u32x4 keep_first(u32x4 x, int v)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (0u - static_cast<uint32_t>(2 * j < v)) & 0x0000FFFFu;
        const uint32_t hi = (0u - static_cast<uint32_t>(2 * j + 1 < v)) & 0xFFFF0000u;
        x[j] &= lo | hi;
    }
    return x;
}

// Resource over the bytes from base (any 2-byte aligned address) to
// base + bytes, widened to whole 16-byte granules: the base is rounded down
// and `mis` returns how many elements it moved.
__device__ inline __amdgpu_buffer_rsrc_t granule_rsrc(const uint16_t *base, int64_t bytes, int &mis)
{
    const uintptr_t p = reinterpret_cast<uintptr_t>(base);
    const uintptr_t al = p & ~static_cast<uintptr_t>(15);
    mis = static_cast<int>((p - al) >> 1);
    const int64_t n = bytes <= 0 ? 0 : ((bytes + static_cast<int64_t>(p - al) + 15) & ~int64_t{15});
    return make_store_rsrc(reinterpret_cast<void *>(al), n);
}

__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <int BT>
__global__ __launch_bounds__(kAnyThreads, 2) void mmrelu_bf16_any(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C, int M, int N, int K,
    int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m, const uint16_t *__restrict__ bias,
    int act)
{
    constexpr int NBLK = BT / 32;                         // 16x16 blocks per wave side
    constexpr int kUnitsA = BT * (kAnyBK / 8);            // 16-byte chunks of an A slab
    constexpr int kUnitsB = kAnyBK * (BT / 8);            // ... of a B slab
    constexpr int kTA = kUnitsA / kAnyThreads, kTB = kUnitsB / kAnyThreads;
    constexpr int kStage = (kUnitsA + kUnitsB) * 8;       // elements per stage
    static_assert(kTA * kAnyThreads == kUnitsA && kTB * kAnyThreads == kUnitsB, "chunk split");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 4, t = lane & 15;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BT, n0 = tn * BT;

    // A: chunk u (one per thread and pass) covers slab row u / 4, k 8q .. +7
    // with q = u % 4 (four consecutive lanes read one row segment, which
    // coalesces best). Its element offset from the rounded-down tile base is
    // r lda + 8q + mis + k0, and k0 is a multiple of 8, so the shift e is
    // fixed for the whole K loop and the slab only adds 2 k0 bytes.
    int a_mis = 0;
    const __amdgpu_buffer_rsrc_t ra =
        granule_rsrc(A + static_cast<int64_t>(m0) * lda, (static_cast<int64_t>(M - 1 - m0) * lda + K) * 2, a_mis);
    uint32_t a_vo[kTA];
    int a_e[kTA];
#pragma unroll
    for (int x = 0; x < kTA; ++x) {
        const int u = x * kAnyThreads + static_cast<int>(threadIdx.x);
        const int r = u >> 2, q = u & 3;
        const int64_t off = static_cast<int64_t>(r) * lda + 8 * q + a_mis;
        a_e[x] = static_cast<int>(off & 7);
        a_vo[x] = m0 + r < M ? static_cast<uint32_t>((off >> 3) * 16) : kOutOfRange;
    }
    // B: chunk u covers slab row u / (BT/8), columns 8 (u % (BT/8)) .. +7.
    // The resource is rebased per slab (B + k0 ldb + n0), so the shifts are
    // recomputed per slab.
    u32x4 pa[kTA][2], pb[kTB][2];
    int b_e[kTB];
    // (The slab offset goes into the per-lane offset, not the scalar one, so
    // that the resource's range check covers the whole address.)
    auto load = [&](int k0) __attribute__((always_inline)) {
        const uint32_t kb = static_cast<uint32_t>(k0) * 2;
#pragma unroll
        for (int x = 0; x < kTA; ++x) {
            const bool ok = a_vo[x] != kOutOfRange;
            pa[x][0] = load16(ra, ok ? a_vo[x] + kb : kOutOfRange, 0);
            pa[x][1] = load16(ra, ok ? a_vo[x] + kb + 16 : kOutOfRange, 0);
        }
        int b_mis = 0;
        const __amdgpu_buffer_rsrc_t rb = granule_rsrc(
            B + static_cast<int64_t>(k0) * ldb + n0, (static_cast<int64_t>(K - 1 - k0) * ldb + N - n0) * 2, b_mis);
#pragma unroll
        for (int x = 0; x < kTB; ++x) {
            const int u = x * kAnyThreads + static_cast<int>(threadIdx.x);
            const int kr = u / (BT / 8), q = u % (BT / 8);
            const int64_t off = static_cast<int64_t>(kr) * ldb + 8 * q + b_mis;
            b_e[x] = static_cast<int>(off & 7);
            const uint32_t vo = k0 + kr < K ? static_cast<uint32_t>((off >> 3) * 16) : kOutOfRange;
            pb[x][0] = load16(rb, vo, 0);
            pb[x][1] = load16(rb, vo == kOutOfRange ? kOutOfRange : vo + 16, 0);
        }
    };
    // Shift, mask and write the loaded slab into stage `buf`.
    auto store = [&](int buf, int k0) __attribute__((always_inline)) {
        uint16_t *st = lds + buf * kStage;
        const bool k_tail = k0 + kAnyBK > K;
#pragma unroll
        for (int x = 0; x < kTA; ++x) {
            const int u = x * kAnyThreads + static_cast<int>(threadIdx.x);
            const int r = u >> 2, q = u & 3;
            u32x4 v = realign(pa[x][0], pa[x][1], a_e[x]);
            if (k_tail) v = keep_first(v, K - k0 - 8 * q);
            *reinterpret_cast<u32x4 *>(st + ((((r >> 4) * 4 + q) * 16) + ((r & 15) ^ (4 * q))) * 8) = v;
        }
        const bool n_tail = n0 + BT > N;
#pragma unroll
        for (int x = 0; x < kTB; ++x) {
            const int u = x * kAnyThreads + static_cast<int>(threadIdx.x);
            const int kr = u / (BT / 8), q = u % (BT / 8);
            u32x4 v = realign(pb[x][0], pb[x][1], b_e[x]);
            if (n_tail) v = keep_first(v, N - n0 - 8 * q);
            *reinterpret_cast<u32x4 *>(st + kUnitsA * 8 + kr * BT + ((q ^ swz_row<BT>(kr)) << 3)) = v;
        }
    };

    // Fragment offsets (elements into a stage). A is chunk-major per 16-row
    // block, as in the aligned kernels, with the row within the block XORed
    // by 4q for chunk q: the 16 lanes that read one chunk still cover one
    // contiguous 256-byte block, and the 16 lanes of a write (rows r .. r+3,
    // chunks 0..3) land on 16 distinct units. A block i: rows
    // wm*BT/2 + 16i + t, chunk g. B block j: lane t of group g reads row
    // 8g + t/4 (+4 for the second half) at columns wn*BT/2 + 16j + 4(t%4) .. +3.
    const int a_off = ((((wm * BT / 2) >> 4) * 4 + g) * 16 + (t ^ (4 * g))) * 8;
    int b_off[NBLK];
    {
        const int k_lane = 8 * g + (t >> 2);
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int n = wn * (BT / 2) + j * 16 + 4 * (t & 3);
            b_off[j] = kUnitsA * 8 + k_lane * BT + (((n >> 3) ^ swz_row<BT>(k_lane)) << 3) + (n & 7);
        }
    }

    f32x4 acc[NBLK][NBLK];
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
        for (int j = 0; j < NBLK; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + kAnyBK - 1) / kAnyBK;
    if (nk > 0) {
        load(0);
        store(0, 0);
    }
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int buf = s & 1;
        if (s + 1 < nk) load((s + 1) * kAnyBK);             // next slab in flight during the MFMAs
        const uint16_t *st = lds + buf * kStage;
        bf16x8 fa[NBLK], fb[NBLK];
#pragma unroll
        for (int i = 0; i < NBLK; ++i) fa[i] = *reinterpret_cast<const bf16x8 *>(st + a_off + i * 16 * kAnyBK);
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            i16x4 half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MMRELU_LDS i16x4 *)(st + b_off[j] + 4 * h * BT));
            fb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < NBLK; ++i)
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        if (s + 1 < nk) store(buf ^ 1, (s + 1) * kAnyBK);   // the other half: last read two slabs ago
        __syncthreads();
    }

    // Epilogue, through LDS. Lane (g, t) of block (i, j) holds C[row t][cols
    // 4g .. 4g+3] of the block; bias and activation on fp32 and one rounding
    // to bf16, then the tile goes to LDS (both stages are free after the
    // loop's last barrier) and each wave stores whole rows of it with the
    // widest stores the row's alignment allows: a row of C may start on any
    // 2-byte boundary, and element-wise stores scattered over sixteen rows
    // cost far more than row-long ones.
    // Tile layout: row r's 8-byte unit u (columns 4u .. 4u+3) at element
    // r BT + 4 ((u + r) % (BT/4)): the sixteen rows of a fragment's lanes
    // start on distinct units, and a row read by BT/4 lanes touches each
    // unit once.
    constexpr int kUnits = BT / 4;                        // 8-byte units per tile row
    constexpr int kRowsPerPass = 64 / kUnits;             // rows one wave covers per store
    static_assert(BT * BT <= 2 * kStage, "the output tile fits in the stages");
    {
        float bj[NBLK][4];
        if (bias != nullptr) {
            const __amdgpu_buffer_rsrc_t rbias = make_bias_rsrc(bias, n0, N, 2);
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) bj[j][r] = bias_bf16(rbias, wn * (BT / 2) + j * 16 + 4 * g + r);
        } else {
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) bj[j][r] = 0.0f;
        }
        with_activation(act, [&](auto act_c) __attribute__((always_inline)) {
            constexpr int ACT = decltype(act_c)::value;
#pragma unroll
            for (int i = 0; i < NBLK; ++i) {
                const int row = wm * (BT / 2) + i * 16 + t;
#pragma unroll
                for (int j = 0; j < NBLK; ++j) {
                    const int u = wn * (BT / 8) + j * 4 + g;
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(activate<ACT>(acc[i][j][r] + bj[j][r]));
                    *reinterpret_cast<u32x2 *>(lds + row * BT + 4 * ((u + row) & (kUnits - 1))) =
                        __builtin_bit_cast(u32x2, o);
                }
            }
        });
    }
    __syncthreads();
    // Wave w stores rows w BT/4 .. (w+1) BT/4 - 1, kRowsPerPass rows a pass;
    // lane l takes row l / kUnits of the pass, columns 4 (l % kUnits) .. +3.
    // A row starting a (mod 4) elements past an 8-byte boundary takes one
    // 8-byte store per lane (a = 0), two 4-byte ones (a = 2), or a 2-, a 4-
    // and a 2-byte one (a odd); a lane with columns past N stores its
    // elements one at a time, those past N not at all; rows past M store
    // nothing (kOutOfRange plus a few bytes is still past every range).
    const int rows = M - m0 < BT ? M - m0 : BT;
    const int ncols = N - n0;
    const __amdgpu_buffer_rsrc_t rc =
        make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0, (static_cast<int64_t>(rows - 1) * ldc + ncols) * 2);
    const int cu = lane & (kUnits - 1);
    const bool full_lane = 4 * cu + 3 < ncols;
    const int a0 = static_cast<int>(((reinterpret_cast<uintptr_t>(C) >> 1) + static_cast<uint64_t>(m0) * ldc + n0) & 3);
    const int ld3 = static_cast<int>(ldc & 3);
#pragma unroll 1
    for (int p = 0; p < BT / 4 / kRowsPerPass; ++p) {
        const int row = wave * (BT / 4) + p * kRowsPerPass + lane / kUnits;
        if (wave * (BT / 4) + p * kRowsPerPass >= rows) break;
        const u32x2 v = *reinterpret_cast<const u32x2 *>(lds + row * BT + 4 * ((cu + row) & (kUnits - 1)));
        const uint32_t off = row < rows ? static_cast<uint32_t>((row * ldc + 4 * cu) * 2) : kOutOfRange;
        const int a = (a0 + row * ld3) & 3;
        if (full_lane) {
            if (a == 0) {
                store_b64(rc, off, v);
            } else if (a == 2) {
                store_b32(rc, off, v[0]);
                store_b32(rc, off + 4, v[1]);
            } else {
                __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v[0]), rc, off, 0, 0);
                store_b32(rc, off + 2, (v[0] >> 16) | (v[1] << 16));
                __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(v[1] >> 16), rc, off + 6, 0, 0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint16_t e = static_cast<uint16_t>((k < 2 ? v[0] : v[1]) >> (16 * (k & 1)));
                __builtin_amdgcn_raw_buffer_store_b16(e, rc, row < rows && 4 * cu + k < ncols ? off + 2 * k : kOutOfRange,
                                                      0, 0);
            }
        }
    }
}

template <int BT>
hipError_t launch_bf16_any(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + BT - 1) / BT, tiles_n = (p.N + BT - 1) / BT;
    hipLaunchKernelGGL(mmrelu_bf16_any<BT>, dim3(static_cast<uint32_t>(grid)), dim3(kAnyThreads), 0, stream,
                       static_cast<const uint16_t *>(p.A), static_cast<const uint16_t *>(p.B),
                       static_cast<uint16_t *>(p.C), p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, 8,
                       static_cast<const uint16_t *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

// 64x64 or 128x128 tiles, any layout.
const Variant *variant_bf16_any(int bt)
{
    static const Variant v64 = {"mmrelu_bf16_any<64,64,32>", MMRELU_DTYPE_BF16, 64, 64, kAnyBK, kAnyThreads, 2, 0,
                                launch_bf16_any<64>, 1.0f};
    static const Variant v128 = {"mmrelu_bf16_any<128,128,32>", MMRELU_DTYPE_BF16, 128, 128, kAnyBK, kAnyThreads, 2, 0,
                                 launch_bf16_any<128>, 1.0f};
    return bt == 64 ? &v64 : &v128;
}

}  // namespace mmrelu
