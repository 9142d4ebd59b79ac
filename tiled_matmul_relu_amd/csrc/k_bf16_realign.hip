// bf16 act(A·B + bias) on the gfx950 matrix cores for any layout, fed by the
// buffer unit's direct global->LDS copies from 4-byte word boundaries.
//
// The lecture's tiled recipe ("Kernels, Triton, XLA", section "Reductions and
// tiling"): one workgroup per output tile, K swept in slabs staged in LDS,
// masked loads that read zeros past the edges, fp32 accumulation, the
// activation on the accumulator, one masked store.
//
// Layouts the 16-byte kernels do not take (odd leading dimensions, N or K not
// multiples of 8, rows that start anywhere on a 2-byte boundary) are staged
// in two steps:
//  * Copy: each operand row's window of the slab is copied from the word
//    boundary at or below the row's first element straight into LDS, 16
//    bytes a lane (buffer_load_dwordx4 ... lds: a dword or longer buffer
//    load needs only 4-byte alignment), or 4 bytes a lane for a slab whose
//    16-byte copy would straddle the end of its operand's range. A row whose
//    first element is the upper half of a word lands one element late: its
//    window holds one element before the slab and lacks the slab's last
//    one, which one more word per such row (its side word) brings in.
//  * Realign: once a slab has landed, the lanes rewrite the late rows in
//    place, each 16-byte chunk joined with the first word of the next chunk
//    (or the side word) and shifted down by one element (v_alignbyte). Rows
//    then sit exactly where the 16-byte kernels put theirs, and the
//    fragment reads are theirs: one ds_read_b128 per A fragment, two
//    ds_read_b64_tr_b16 per B fragment.
// Whether a row is late depends on the row only (slabs start at multiples of
// 32 elements, so k0 * ld is even): the plan is made once per tile.
//
// Tile BM x 256 per workgroup of eight waves (2 x 4), each a BM/2 x 64
// sub-tile of BM/32 x 4 blocks of v_mfma_f32_16x16x32_bf16 (up to 128 fp32
// accumulators per lane); K in slabs of 32 in a ring of four LDS stages. In
// step kt every wave multiplies slab kt (fragments in registers), reads slab
// kt+1's fragments, realigns slab kt+2 and issues the copies of slab kt+4
// into the stage slab kt left; one barrier per step. Every wave both
// multiplies and moves data, so a step lasts as long as each wave's own mix
// of MFMAs, fragment reads, realign round trip and copy issue, which the two
// waves of a SIMD, in the same phase, hide only in part: the copies of inner
// slabs (all but the last few) carry no per-lane tests, only late rows are
// realigned, and each realign's write comes two parts after its read. This
// schedule reaches 0.24-0.45 of the bf16 peak, against about
// 0.6 for the ping-pong kernels, whose two wave groups take the two roles in
// turn but need 16-byte aligned rows.
//
// BM is 256, 224, 192 or 160: the shorter tiles give shapes whose 256-row
// grid would leave CUs idle more tiles of less work each (4097 x 3001: 204
// tiles of 256 rows, 228 of 224). Copies and realign always cover 256 rows;
// rows past BM belong to the next tile and are staged but not multiplied.
//
// LDS stage (34 KB): A, 256 rows x 64 bytes, chunk c of row r at r*64 +
// 16 (c ^ (r/2 % 4)); B, 32 rows x 512 bytes, chunk c of row k at k*512 +
// 16 (c ^ swz_b(k)); then the side words, A's (one per row) and B's (one per
// slab row). A 16-byte copy fills 1 KB (16 A rows or 2 B rows), a 4-byte
// copy 256 bytes; wave w fills the same bytes either way.
//
// Edges: rows past M and B rows past K get out-of-range offsets (the copy
// writes zeros); A elements past K in the last slab are zeroed while
// realigning (the words there hold the next row's elements); B columns past N
// hold whatever follows in memory and only reach outputs past N, which are
// never stored. Each resource ends at the word that holds the operand's last
// element, and a 4-byte word never crosses a page, so the bytes read around
// an operand are always mapped. The output tile is staged in LDS and stored
// in whole rows, each with the widest stores its alignment allows, so any
// ldc works.
#include <type_traits>

#include "kernels.hpp"
#include "device_common.hpp"
#include "../../include/mmrelu.h"

namespace mmrelu {
namespace {

constexpr int kTile = 256, kSlab = 32, kThreads = 512, kStages = 4;
constexpr int kNB = 4;                                   // MFMA column blocks per wave: 64 columns
constexpr int kABytes = kTile * kSlab * 2;               // A part of a stage
constexpr int kBBytes = kSlab * kTile * 2;               // B part
constexpr int kSideA = kABytes + kBBytes;                // A's side words, one per tile row
constexpr int kSideB = kSideA + kTile * 4;               // B's side words, one per slab row
constexpr int kStageBytes = kSideA + 8 * 256;            // side block: one 256-byte copy per wave
static_assert(kStages * kStageBytes <= 160 * 1024, "LDS budget");

__device__ inline int swz_b(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }
// A's 64-byte rows: chunk c of row r at r*64 + 16 (c ^ (r/2 % 4)). Eight
// lanes reading one chunk of eight consecutive rows (a fragment read) then
// touch eight distinct 16-byte slots of each 128-byte bank window.
__device__ inline uint32_t a_byte(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }
__device__ inline uint32_t b_byte(int k, int c) { return kABytes + k * 512 + 16 * (c ^ swz_b(k)); }

// The 8 elements that start one element into the 18 bytes lo:next (element
// j of the result is element j+1 of the pair).
__device__ inline u32x4 shift_down(const u32x4 &lo, uint32_t next)
{
    u32x4 out;
    out[0] = __builtin_amdgcn_alignbyte(lo[1], lo[0], 2);
    out[1] = __builtin_amdgcn_alignbyte(lo[2], lo[1], 2);
    out[2] = __builtin_amdgcn_alignbyte(lo[3], lo[2], 2);
    out[3] = __builtin_amdgcn_alignbyte(next, lo[3], 2);
    return out;
}

// Keep the first v of the 8 elements in x (v <= 0: none), zero the rest.
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

template <int BM>
__global__ __launch_bounds__(kThreads, 1) void mmrelu_bf16_realign(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, uint16_t *__restrict__ C, int M, int N, int K,
    int64_t lda, int64_t ldb, int64_t ldc, int tiles_m, int tiles_n, int group_m, const uint16_t *__restrict__ bias,
    int act)
{
    static_assert(BM % 32 == 0 && BM >= 160 && BM <= kTile, "tile rows");
    constexpr int kMB = BM / 32;                          // MFMA row blocks per wave: BM/2 rows
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStageBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int g = lane >> 4, t = lane & 15;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * kTile;
    const int rows = M - m0;                              // rows of A and C from m0 on (may exceed BM)
    const uint32_t lds0 = lds_address(lds);

    // Word bases. Row r of the tile starts a_mis + r lda elements past A's
    // word base; row k of slab k0, b_mis + k ldb past the word base of B's
    // slab (k0 ldb is even, so b_mis is the same for every slab).
    const uintptr_t a_addr = reinterpret_cast<uintptr_t>(A + static_cast<int64_t>(m0) * lda);
    const uintptr_t b_addr = reinterpret_cast<uintptr_t>(B + n0);
    const int a_mis = static_cast<int>((a_addr >> 1) & 1), b_mis = static_cast<int>((b_addr >> 1) & 1);
    // Byte ranges of the A resource and of the B resource of slab k0: up to
    // the word that holds the operand's last element.
    const int64_t a_range = ((a_mis + static_cast<int64_t>(rows - 1) * lda + K) * 2 + 3) & ~int64_t{3};
    auto b_range = [&](int k0) {
        return ((b_mis + static_cast<int64_t>(K - 1 - k0) * ldb + N - n0) * 2 + 3) & ~int64_t{3};
    };
    const rsrc_t ra = make_rsrc(reinterpret_cast<const void *>(a_addr & ~uintptr_t{3}), a_range);
    // First word of row r's window (byte offset from the word base, k0 = 0),
    // and whether the row is late.
    auto a_word0 = [&](int r) { return static_cast<uint32_t>(((a_mis + static_cast<int64_t>(r) * lda) >> 1) * 4); };
    auto a_late = [&](int r) { return ((a_mis + static_cast<int64_t>(r) * lda) & 1) != 0; };
    auto b_word0 = [&](int k) { return static_cast<uint32_t>(((b_mis + static_cast<int64_t>(k) * ldb) >> 1) * 4); };
    auto b_late = [&](int k) { return ((b_mis + static_cast<int64_t>(k) * ldb) & 1) != 0; };

    // Copy plans. A copy moves 16 bytes a lane (1 KB an instruction) from
    // any 4-byte boundary (buffer loads of a dword or more need only 4-byte
    // alignment), or, near the end of an operand, 4 bytes a lane: a 16-byte
    // copy that would straddle the end of its resource's range is never
    // issued (see `copy_edge`). Either way wave w fills the same LDS bytes.
    //  A copy q (0, 1) of wave w fills rows 128q + 16w + l/4, stored chunk
    //  l%4 = the row's chunk l%4 ^ (l/8 % 4); row 128q + r's window starts
    //  256 q lda bytes after row r's. As four 4-byte copies d = 0..3, copy d
    //  fills rows 128q + 16w + 4d + l/16, stored chunk (l/4)%4, the row's
    //  chunk (l/4)%4 ^ ((2d + l/32) % 4), word l%4.
    //  B copy q fills slab rows 16q + 2w + l/32, stored chunk l%32 = the
    //  row's chunk l%32 ^ swz_b(row), where swz_b(16q + r) = swz_b(r); row
    //  16q + r's window starts 32 q ldb bytes after row r's. As four 4-byte
    //  copies, copy d fills half d%2 of row 16q + 2w + d/2: stored chunk
    //  16 (d%2) + l/4, word l%4.
    //  Side words: wave w's block holds words 64w .. 64w+63; words 0-255 are
    //  A rows' (word 16 of the window), 256-287 B slab rows' (word 128).
    const bool side_b = wave == 4;
    const int nk = (K + kSlab - 1) / kSlab;
    auto ax_row = [&](int l) __attribute__((always_inline)) { return 16 * wave + (l >> 2); };
    auto ax_plan = [&](int l) __attribute__((always_inline)) { return a_word0(ax_row(l)) + 16 * ((l & 3) ^ ((l >> 3) & 3)); };
    auto bx_row = [&](int l) __attribute__((always_inline)) { return 2 * wave + (l >> 5); };
    auto bx_plan = [&](int l) __attribute__((always_inline)) { return b_word0(bx_row(l)) + 16 * ((l & 31) ^ swz_b(bx_row(l))); };
    auto side_plan = [&](int l) __attribute__((always_inline)) {
        // Both candidates are computed and one selected (a branch here let
        // the compiler select between the addresses of lda and ldb, which
        // put them in scratch memory).
        const int sd = 64 * wave + l, kb = sd - kTile;
        const uint32_t va = a_word0(sd) + 64, vb = b_word0(kb) + 512;
        const bool ok_a = sd < kTile && sd < rows && a_late(sd);
        const bool ok_b = sd >= kTile && kb < kSlab && b_late(kb);
        return ok_a ? va : (ok_b ? vb : kOutOfRange);
    };
    // Inner slabs. Every 16-byte copy of a slab with k0 + 32 <= K ends
    // inside A's range: row r's window ends at most (r lda + k0 + 32) * 2
    // bytes past the base, and the range at ((rows-1) lda + K) * 2. Its B
    // rows all lie inside K, and row k's window ends at most (k ldb + 256) *
    // 2 bytes past the slab's base, against ((K-1-k0) ldb + N - n0) * 2 for
    // the range: inside it whenever (K - 32 - k0) ldb >= 256 - (N - n0),
    // which b_slack turns into a count of slabs. For such slabs the copies
    // need no tests at all: the only per-lane condition left, rows past M,
    // is folded into the A offsets once per tile.
    // (Per-tile values from 64-bit divisions are computed on the vector
    // unit; readfirstlane puts them back in scalar registers.)
    const int b_slack = __builtin_amdgcn_readfirstlane(
        N - n0 >= kTile ? 0 : static_cast<int>((kTile - (N - n0) + ldb - 1) / ldb));
    auto inner_slab = [&](int s) __attribute__((always_inline)) { return s * kSlab + kSlab + b_slack <= K; };
    uint32_t in_ax0, in_ax1, in_bx, in_side;
    {
        const uint32_t a0 = ax_plan(lane);
        in_ax0 = ax_row(lane) < rows ? a0 : kOutOfRange;
        in_ax1 = ax_row(lane) + 128 < rows ? a0 + static_cast<uint32_t>(256 * lda) : kOutOfRange;
        in_bx = bx_plan(lane);
        in_side = side_plan(lane);
    }
    // Resource of B's slab at k0 = 32 s: the base moves by 64 ldb bytes a
    // slab (a multiple of 4, so the word alignment below the row start is
    // the same for every slab) and the range shrinks by as much.
    const uintptr_t b_base0 = b_addr & ~uintptr_t{3};
    const int64_t b_range0 = b_range(0);
    auto b_rsrc_slab = [&](int s) __attribute__((always_inline)) {
        const int64_t step = static_cast<int64_t>(s) * 64 * ldb;
        return make_rsrc(reinterpret_cast<const void *>(b_base0 + static_cast<uintptr_t>(step)), b_range0 - step);
    };
    // The same for an inner slab, whose range is positive: kMaxRange until
    // slab s_small, where it first falls below that, and from there on the
    // low 32 bits of b_range0 - step (scalar 32-bit arithmetic only).
    const int64_t b_over = b_range0 - kMaxRange;
    const int s_small = __builtin_amdgcn_readfirstlane(
        b_over <= 0 ? 0 : static_cast<int>((b_over + 64 * ldb - 1) / (64 * ldb)));
    auto b_rsrc_inner = [&](int s) __attribute__((always_inline)) {
        const uint64_t step = static_cast<uint64_t>(s) * 64 * static_cast<uint64_t>(ldb);
        const uint64_t a = b_base0 + step;
        const uint32_t range = s >= s_small ? static_cast<uint32_t>(b_range0) - static_cast<uint32_t>(step)
                                            : static_cast<uint32_t>(kMaxRange);
        rsrc_t r;
        r[0] = static_cast<int32_t>(a);
        r[1] = static_cast<int32_t>((a >> 32) & 0xFFFF);
        r[2] = static_cast<int32_t>(range);
        r[3] = static_cast<int32_t>(kBufferFormat);
        return r;
    };
    // Copies of an inner slab, five per wave: q = 0, 1 for A, 2, 3 for B,
    // 4 for the side words.
    auto copy_inner_q = [&](int s, int q, rsrc_t rb) __attribute__((always_inline)) {
        const int k0 = s * kSlab;
        const uint32_t st = lds0 + (s & (kStages - 1)) * kStageBytes;
        if (q == 0) load_to_lds_z<16>(ra, st + wave * 1024, in_ax0 + 2 * k0);
        if (q == 1) load_to_lds_z<16>(ra, st + (8 + wave) * 1024, in_ax1 + 2 * k0);
        if (q == 2) load_to_lds_z<16>(rb, st + kABytes + wave * 1024, in_bx);
        if (q == 3) load_to_lds_z<16>(rb, st + kABytes + (8 + wave) * 1024, in_bx + static_cast<uint32_t>(32 * ldb));
        if (q == 4) {
            if (side_b) load_to_lds_z<4>(rb, st + kSideA + wave * 256, in_side);
            else load_to_lds_z<4>(ra, st + kSideA + wave * 256, in_side + 2 * k0);
        }
    };
    auto copy_inner = [&](int s, rsrc_t rb) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 5; ++q) copy_inner_q(s, q, rb);
    };
    // Copies of an edge slab (the last slabs, and slabs past K, which copy
    // zeros): every copy tested against M and K, and the whole slab copied
    // 4 bytes a lane if one of the wave's 16-byte copies would straddle the
    // end of its range (every 4-byte word is wholly in range or wholly out).
    // The plan is derived from the lane id again here, through an asm the
    // compiler cannot see through, so none of it stays live across the loop.
    constexpr int kCopiesWide = 5;                       // 16-byte copies per wave per slab (17 when 4-byte)
    auto copy_edge = [&](int s, rsrc_t rb) __attribute__((always_inline)) {
        int l = lane;
        asm volatile("" : "+v"(l));
        const int ar = ax_row(l), br = bx_row(l);
        const uint32_t ax = ax_plan(l), bx = bx_plan(l), side = side_plan(l);
        const bool live = s < nk;
        const int k0 = s * kSlab;
        const uint32_t st = lds0 + (s & (kStages - 1)) * kStageBytes;
        const int64_t rb_end = b_range(k0);
        bool r = false;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t oa = static_cast<int64_t>(ax) + 256 * q * lda + 2 * k0;
            r |= ar + 128 * q < rows && oa < a_range && oa + 16 > a_range;
            const int64_t ob = static_cast<int64_t>(bx) + 32 * q * ldb;
            r |= k0 + br + 16 * q < K && ob < rb_end && ob + 16 > rb_end;
        }
        if (!(live && __builtin_amdgcn_ballot_w64(r) != 0)) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const bool ok = live && ar + 128 * q < rows;
                const uint32_t off = ax + static_cast<uint32_t>(256 * q * lda + 2 * k0);
                load_to_lds<16>(ra, st + (8 * q + wave) * 1024, ok ? off : kOutOfRange);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const bool ok = live && k0 + br + 16 * q < K;
                const uint32_t off = bx + static_cast<uint32_t>(32 * q * ldb);
                load_to_lds<16>(rb, st + kABytes + (8 * q + wave) * 1024, ok ? off : kOutOfRange);
            }
        } else {
            const int an_row = 16 * wave + (l >> 4);
            const uint32_t an = a_word0(an_row) + 4 * (l & 3);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const bool ok = an_row + 128 * c + 4 * d < rows;
                    const uint32_t off = an + static_cast<uint32_t>((256 * c + 8 * d) * lda + 2 * k0) +
                                         16 * (((l >> 2) & 3) ^ ((2 * d + (l >> 5)) & 3));
                    load_to_lds<4>(ra, st + (8 * c + wave) * 1024 + 256 * d, ok ? off : kOutOfRange);
                }
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int row = 2 * wave + (d >> 1);         // of the slab, less 16 c
                    const bool ok = k0 + row + 16 * c < K;
                    const uint32_t off = b_word0(row) + static_cast<uint32_t>(32 * c * ldb) +
                                         16 * ((16 * (d & 1) + (l >> 2)) ^ swz_b(row)) + 4 * (l & 3);
                    load_to_lds<4>(rb, st + kABytes + (8 * c + wave) * 1024 + 256 * d, ok ? off : kOutOfRange);
                }
        }
        const bool ok = live && side != kOutOfRange && (!side_b || k0 + l < K);
        const uint32_t off = side_b ? side : side + static_cast<uint32_t>(2 * k0);
        load_to_lds<4>(side_b ? rb : ra, st + kSideA + wave * 256, ok ? off : kOutOfRange);
    };
    auto issue_slab = [&](int s) __attribute__((always_inline)) {
        const rsrc_t rb = b_rsrc_slab(s);
        if (inner_slab(s)) copy_inner(s, rb);
        else copy_edge(s, rb);
    };

    // Realign plan: the late rows of a slab. With an odd leading dimension
    // every other row is late, and one unit per lane covers them: A row
    // 2 ((64w + l) / 4) + pa, chunk l%4, and B row 2 ((64w + l) / 32) + pb,
    // chunk l%32 (pa, pb = 1 when row 0 is not late). With an even one
    // every row is late or none is, and a lane has two units: A rows 32w +
    // 16j + l/4 (j = 0, 1), B rows 4w + 2j + l/32. A unit joins its chunk
    // with the next chunk's first word, or with the side word for the last
    // chunk. A row's chunks sit in consecutive lanes of one wave, so every
    // next word is read before any chunk of the row is rewritten.
    const bool a_alt = (lda & 1) != 0, b_alt = (ldb & 1) != 0;
    const int a_units = a_alt ? 1 : (a_late(0) ? 2 : 0);
    const int b_units = b_alt ? 1 : (b_late(0) ? 2 : 0);
    const int ra_row = a_alt ? 2 * ((64 * wave + lane) >> 2) + (a_late(0) ? 0 : 1) : 32 * wave + (lane >> 2);
    const int ra_c = lane & 3;
    const uint32_t ra_main = a_byte(ra_row, ra_c);                                 // + 1024 j
    const uint32_t ra_next = ra_c < 3 ? a_byte(ra_row, ra_c + 1) : kSideA + 4 * ra_row;
    const uint32_t ra_step = ra_c < 3 ? 1024u : 64u;
    const int rb_row = b_alt ? 2 * ((64 * wave + lane) >> 5) + (b_late(0) ? 0 : 1) : 4 * wave + (lane >> 5);
    const int rb_c = lane & 31;
    uint32_t rb_main[2], rb_next[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        rb_main[j] = b_byte(rb_row + 2 * j, rb_c);
        rb_next[j] = rb_c < 31 ? b_byte(rb_row + 2 * j, rb_c + 1) : kSideB + 4 * (rb_row + 2 * j);
    }
    // An operand without late rows has the main loop realign garbage in a
    // spare part of the stage instead, so that its steps need no test: side
    // words 288-511 are written (with zeros) by copies into the stage and
    // read by nothing else.
    const uint32_t dummy = kSideA + 4 * (kTile + kSlab) + 16 * (lane & 31);
    static_assert(kSideA + 4 * (kTile + kSlab) + 16 * 32 <= kStageBytes, "spare side words");
    const uint32_t ra_main_f = a_units > 0 ? ra_main : dummy, ra_next_f = a_units > 0 ? ra_next : dummy;
    const uint32_t rb_main_f = b_units > 0 ? rb_main[0] : dummy, rb_next_f = b_units > 0 ? rb_next[0] : dummy;
    // The slab that holds K's end (or lies past it): every A row, late or
    // not, has its elements past K zeroed (rows 32w + 16j + l/4, chunk
    // l%4), and B's late rows are realigned as in any slab.
    auto realign_tail = [&](int s) __attribute__((always_inline)) {
        uint8_t *st = lds + (s & (kStages - 1)) * kStageBytes;
        const int k0 = s * kSlab;
        const int tr = 32 * wave + (lane >> 2);
        const bool t_late = a_late(tr);
        const uint32_t t_main = a_byte(tr, ra_c);
        const uint32_t t_next = ra_c < 3 ? a_byte(tr, ra_c + 1) : kSideA + 4 * tr;
        u32x4 v[2];
        uint32_t x[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            v[j] = *reinterpret_cast<const u32x4 *>(st + t_main + 1024 * j);
            x[j] = *reinterpret_cast<const uint32_t *>(st + t_next + ra_step * j);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (t_late) v[j] = shift_down(v[j], x[j]);
            *reinterpret_cast<u32x4 *>(st + t_main + 1024 * j) = keep_first(v[j], K - k0 - 8 * ra_c);
        }
        if (b_units > 0) {
            u32x4 w[2];
            uint32_t y[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (j < b_units) {
                    w[j] = *reinterpret_cast<const u32x4 *>(st + rb_main[j]);
                    y[j] = *reinterpret_cast<const uint32_t *>(st + rb_next[j]);
                }
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (j < b_units) *reinterpret_cast<u32x4 *>(st + rb_main[j]) = shift_down(w[j], y[j]);
        }
    };
    // Any other slab, in two halves so that the LDS round trip can be
    // covered by MFMAs: realign_read(s, u) loads unit u of this lane's A and
    // B late rows into registers, realign_write(s, u) shifts and stores them.
    u32x4 rl_va, rl_vb;
    uint32_t rl_xa, rl_xb;
    auto realign_read = [&](int s, int u) __attribute__((always_inline)) {
        const uint8_t *st = lds + (s & (kStages - 1)) * kStageBytes;
        if (u < a_units) {
            rl_va = *reinterpret_cast<const u32x4 *>(st + ra_main + 1024 * u);
            rl_xa = *reinterpret_cast<const uint32_t *>(st + ra_next + ra_step * u);
        }
        if (u < b_units) {
            rl_vb = *reinterpret_cast<const u32x4 *>(st + rb_main[u]);
            rl_xb = *reinterpret_cast<const uint32_t *>(st + rb_next[u]);
        }
    };
    auto realign_write = [&](int s, int u) __attribute__((always_inline)) {
        uint8_t *st = lds + (s & (kStages - 1)) * kStageBytes;
        if (u < a_units) *reinterpret_cast<u32x4 *>(st + ra_main + 1024 * u) = shift_down(rl_va, rl_xa);
        if (u < b_units) *reinterpret_cast<u32x4 *>(st + rb_main[u]) = shift_down(rl_vb, rl_xb);
    };
    // The main loop's form: one unit of each operand, real or in the spare
    // side words, with no test.
    auto realign_read_f = [&](int s) __attribute__((always_inline)) {
        const uint8_t *st = lds + (s & (kStages - 1)) * kStageBytes;
        rl_va = *reinterpret_cast<const u32x4 *>(st + ra_main_f);
        rl_xa = *reinterpret_cast<const uint32_t *>(st + ra_next_f);
        rl_vb = *reinterpret_cast<const u32x4 *>(st + rb_main_f);
        rl_xb = *reinterpret_cast<const uint32_t *>(st + rb_next_f);
    };
    auto realign_write_f = [&](int s) __attribute__((always_inline)) {
        uint8_t *st = lds + (s & (kStages - 1)) * kStageBytes;
        *reinterpret_cast<u32x4 *>(st + ra_main_f) = shift_down(rl_va, rl_xa);
        *reinterpret_cast<u32x4 *>(st + rb_main_f) = shift_down(rl_vb, rl_xb);
    };
    // Two units per lane (even leading dimensions with every row late) are
    // done in full when first reached; one unit (odd ones) may be written
    // some parts after it is read.
    const bool rl_two = a_units == 2 || b_units == 2;
    auto is_tail = [&](int s) __attribute__((always_inline)) { return K - s * kSlab < kSlab; };
    auto realign = [&](int s) __attribute__((always_inline)) {
        if (is_tail(s)) {
            realign_tail(s);
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                realign_read(s, u);
                realign_write(s, u);
            }
        }
    };

    // Fragment reads. A block i: rows wm*BM/2 + 16i + t, chunk g; B block j:
    // lane t of group g addresses slab row 8g + t/4 (+4 for the second
    // half) at columns wn*64 + 16j + 4(t%4) .. +3.
    const uint32_t a_frag = a_byte(wm * (BM / 2) + t, g);                         // + 1024 i
    uint32_t b_frag[kNB];
    {
        const int k_lane = 8 * g + (t >> 2);
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int n = wn * 64 + j * 16 + 4 * (t & 3);
            b_frag[j] = b_byte(k_lane, n >> 3) + 2 * (n & 7);
        }
    }
    // A fragments are held once: block i of slab kt+1 is read right after
    // the four MFMAs of slab kt that use block i. B fragments are held twice
    // (slab kt's are used by every A block): fb, and fb_next for slab kt+1;
    // the main loop runs two steps at a time with the two sets swapping
    // roles, the other steps hand fb_next over to fb (16 moves).
    bf16x8 fa[kMB], fb[kNB], fb_next[kNB];
    auto load_frag_a = [&](int s, int i) __attribute__((always_inline)) {
        const uint8_t *st = lds + (s & (kStages - 1)) * kStageBytes;
        fa[i] = *reinterpret_cast<const bf16x8 *>(st + a_frag + 1024 * i);
    };
    auto load_frag_b = [&](bf16x8 &dst, int s, int j) __attribute__((always_inline)) {
        const uint8_t *st = lds + (s & (kStages - 1)) * kStageBytes;
        i16x4 half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MMRELU_LDS i16x4 *)(st + b_frag[j] + 4 * 512 * h));
        dst = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };

    f32x4 acc[kMB][kNB];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfma_row_with = [&](int i, const bf16x8 (&b)[kNB]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kNB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], fa[i], acc[i][j], 0, 0, 0);
    };
    auto mfma_row = [&](int i) __attribute__((always_inline)) { mfma_row_with(i, fb); };

    // Step kt (slab kt+1 exists): wait for slab kt+2 (slab kt+3 may stay in
    // flight; waiting for all but the 16-byte count of one slab over-waits
    // after a slab of 4-byte copies, which is harmless), barrier; then BM/32
    // parts, one per A block i: the four MFMAs of block i of slab kt, the
    // read of block i of slab kt+1 and, in four of the parts (every other
    // one for 256 rows), one B fragment of slab kt+1. Between parts, while
    // the matrix cores work through the MFMAs issued so far: after part 0
    // the late rows of slab kt+2 are read; after part 2 (part 1 in the last
    // steps) they are written back realigned, two parts of MFMAs hiding the
    // read's latency (written after part 1: 4097x3001x2049 68.6 against
    // 67.0 us, 3001^3 92.3 against 87.4); and after parts 1-5 (the last part
    // taking the rest when there are fewer) the five copies of slab kt+4
    // (into slab kt's stage) are issued one at a time (an edge slab's all
    // after part 1). One at a time, a copy holds up the wave's next MFMAs
    // for less (4097x3001x2049: 91.7 against 95.4 us with the copies
    // together and the realign in one part). The fences keep each part's
    // MFMAs inside the part, ahead of the read that overwrites their operand.
    // kFast: a step whose copies are of an inner slab and whose realign is
    // of a whole slab with at most one late unit per lane (all steps but the
    // last few, with an odd leading dimension or no late rows); its tests
    // are then compile-time constants and its parts carry no branches.
    auto step = [&](int kt, auto fast_c, bf16x8 (&cur)[kNB], bf16x8 (&nxt)[kNB], bool hand_over)
                    __attribute__((always_inline)) {
        constexpr bool kFast = decltype(fast_c)::value;
        const bool rl = kFast || kt + 2 < nk, rl_tail = !kFast && rl && is_tail(kt + 2);
        const bool inner = kFast || inner_slab(kt + 4);
        const bool two = !kFast && rl_two;
        rsrc_t rb_step;
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kCopiesWide>();
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
            mfma_row_with(i, cur);
            load_frag_a(kt + 1, i);
#pragma unroll
            for (int j = 0; j < kNB; ++j)
                if (i == j * kMB / kNB) load_frag_b(nxt[j], kt + 1, j);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two MFMAs
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // the LDS reads
            __builtin_amdgcn_sched_barrier(0);
            if (kFast) {
                if (i == 0) realign_read_f(kt + 2);
                if (i == 2) realign_write_f(kt + 2);
            } else {
                if (i == 0 && rl) {
                    if (rl_tail || two) realign(kt + 2);
                    else realign_read(kt + 2, 0);
                }
                if (i == 1 && rl && !rl_tail && !two) realign_write(kt + 2, 0);
            }
            if (inner) {
                if (i == 1) rb_step = kFast ? b_rsrc_inner(kt + 4) : b_rsrc_slab(kt + 4);
#pragma unroll
                for (int q = 0; q < 5; ++q)
                    if (i == (1 + q < kMB - 1 ? 1 + q : kMB - 1)) copy_inner_q(kt + 4, q, rb_step);
            } else if (i == 1) {
                issue_slab(kt + 4);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (hand_over)
#pragma unroll
            for (int j = 0; j < kNB; ++j) cur[j] = nxt[j];
    };
    if (nk > 0) {
        issue_slab(0);
        issue_slab(1);
        issue_slab(2);
        wait_vmcnt<kCopiesWide>();                        // slabs 0 and 1 have landed
        __syncthreads();
        realign(0);
        if (nk > 1) realign(1);
        issue_slab(3);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kNB; ++j) load_frag_b(fb[j], 0, j);
#pragma unroll
        for (int i = 0; i < kMB; ++i) load_frag_a(0, i);
        int kt = 0;
        if (!rl_two)
            for (; inner_slab(kt + 5); kt += 2) {
                step(kt, std::true_type{}, fb, fb_next, false);
                step(kt + 1, std::true_type{}, fb_next, fb, false);
            }
        for (; kt + 1 < nk; ++kt) step(kt, std::false_type{}, fb, fb_next, true);
#pragma unroll
        for (int i = 0; i < kMB; ++i) mfma_row(i);
        wait_vmcnt<0>();                                  // the zero fills past K
    }

    // Epilogue, through LDS. Lane (g, t) of block (i, j) holds C[row][col ..
    // col+3]; bias and activation on fp32 and one rounding to bf16, then the
    // tile goes to LDS (the stages are free once every copy has landed) and
    // each wave stores whole rows of it with the widest stores the row's
    // alignment allows: a row of C may start on any 2-byte boundary, and a
    // row written 2 bytes a lane at a time costs far more than the same
    // bytes in row-long stores (4097x3001x2049: 17 of 83 us).
    // Tile layout: row r's 8-byte unit u (columns 4u .. 4u+3) at r*512 +
    // 8 ((u + 4r) % 64). The sixteen rows and four units of a fragment's
    // lanes fall on distinct bank pairs, and a row read by 64 lanes touches
    // each unit once.
    __syncthreads();
    {
        float bj[kNB][4];
        if (bias != nullptr) {
            const __amdgpu_buffer_rsrc_t rbias = make_bias_rsrc(bias, n0, N, 2);
#pragma unroll
            for (int j = 0; j < kNB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) bj[j][r] = bias_bf16(rbias, wn * 64 + j * 16 + 4 * g + r);
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
                const int row = wm * (BM / 2) + i * 16 + t;
#pragma unroll
                for (int j = 0; j < kNB; ++j) {
                    const int u = wn * 16 + j * 4 + g;
                    bf16x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = static_cast<__bf16>(activate<ACT>(acc[i][j][r] + bj[j][r]));
                    *reinterpret_cast<u32x2 *>(lds + row * 512 + 8 * ((u + 4 * row) & 63)) =
                        __builtin_bit_cast(u32x2, o);
                }
            }
        });
    }
    __syncthreads();
    // Wave w stores rows w BM/8 .. (w+1) BM/8 - 1 (those below M); lane l columns 4l ..
    // 4l+3. A row starting a (mod 4) elements past an 8-byte boundary takes
    // one 8-byte store per lane (a = 0), two 4-byte ones (a = 2), or a 2-,
    // a 4- and a 2-byte one (a odd); a lane with columns past N stores its
    // elements one at a time, those past N not at all.
    const __amdgpu_buffer_rsrc_t rc =
        make_store_rsrc(C + static_cast<int64_t>(m0) * ldc + n0, (static_cast<int64_t>(rows - 1) * ldc + N - n0) * 2);
    const int ncols = N - n0;
    const bool full_lane = 4 * lane + 3 < ncols;
    const int a0 = static_cast<int>(((reinterpret_cast<uintptr_t>(C) >> 1) + static_cast<uint64_t>(m0) * ldc + n0) & 3);
    const int ld3 = static_cast<int>(ldc & 3);
#pragma unroll 1
    for (int rr = 0; rr < BM / 8; ++rr) {
        const int row = BM / 8 * wave + rr;
        if (row >= rows) break;
        const u32x2 v = *reinterpret_cast<const u32x2 *>(lds + row * 512 + 8 * ((lane + 4 * row) & 63));
        const uint32_t off = static_cast<uint32_t>((row * ldc + 4 * lane) * 2);
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
                __builtin_amdgcn_raw_buffer_store_b16(e, rc, 4 * lane + k < ncols ? off + 2 * k : kOutOfRange, 0, 0);
            }
        }
    }
}

// Tile-row bands of this height are walked column by column inside each
// XCD's range of tiles (tile_of).
constexpr int kGroupM = 8;

template <int BM>
hipError_t launch_realign(const Problem &p, int64_t grid, hipStream_t stream)
{
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + kTile - 1) / kTile;
    hipLaunchKernelGGL(mmrelu_bf16_realign<BM>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t *>(p.A), static_cast<const uint16_t *>(p.B),
                       static_cast<uint16_t *>(p.C), p.M, p.N, p.K, p.lda, p.ldb, p.ldc, tiles_m, tiles_n, kGroupM,
                       static_cast<const uint16_t *>(p.bias), p.act);
    return hipGetLastError();
}

}  // namespace

// BM x 256 tiles (BM = 256, 224, 192 or 160), any layout.
const Variant *variant_bf16_realign(int bm)
{
    static const Variant v256 = {"mmrelu_bf16_realign<256,256,32>", MMRELU_DTYPE_BF16, 256, kTile, kSlab, kThreads,
                                 1, 0, launch_realign<256>, 1.0f};
    static const Variant v224 = {"mmrelu_bf16_realign<224,256,32>", MMRELU_DTYPE_BF16, 224, kTile, kSlab, kThreads,
                                 1, 0, launch_realign<224>, 1.0f};
    static const Variant v192 = {"mmrelu_bf16_realign<192,256,32>", MMRELU_DTYPE_BF16, 192, kTile, kSlab, kThreads,
                                 1, 0, launch_realign<192>, 1.0f};
    static const Variant v160 = {"mmrelu_bf16_realign<160,256,32>", MMRELU_DTYPE_BF16, 160, kTile, kSlab, kThreads,
                                 1, 0, launch_realign<160>, 1.0f};
    return bm == 224 ? &v224 : bm == 192 ? &v192 : bm == 160 ? &v160 : &v256;
}

}  // namespace mmrelu
