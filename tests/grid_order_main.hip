// Host check of the dealt grid order (dealt_tile, causal_deal, make_deal in
// cdna4.h): for the launch shapes of the dense causal forwards,
// the causal backward's dQ and dK/dV grids and varlen batches (unequal
// lengths, and causal ones of nearly equal lengths), every workgroup id of the grid
// maps to padding or to one (head, query tile) in range, and every (head,
// query tile) is reached exactly once, and the XCDs receive equal causal
// work up to a few of a group's lightest tiles.  The launches use two tile
// forms: 256-row tiles and 32 slots per XCD (8-wave workgroups), or 128-row
// tiles and 64 slots (4-wave workgroups: bf16 grids too small for the 8-wave
// form, short sequences, narrow windows, and FP8 always); every shape is
// checked in both forms.
// Prints "ok ..." and exits 0, or names the first failing shape and exits 1.
#include "cdna4.h"

#include <cstdio>
#include <vector>

using namespace cdna4;

static long n_shapes = 0, n_dealt = 0;

static int64_t worst_gap = 0;

static bool covers(int64_t per, int64_t G, int64_t n, const Deal& d, int64_t grid, const char* what,
                   long a, long b, long c) {
    std::vector<uint8_t> seen((size_t)(per * n), 0);
    int64_t hits = 0;
    int64_t work[8] = {0};   // causal work per XCD: tile qt sees qt + 1 diagonal-width key blocks
    for (int64_t bid = 0; bid < grid; ++bid) {
        int bh = -1, qt = -1;
        if (!dealt_tile((int)bid, (int)per, (int)G, (int)n, d, bh, qt)) continue;
        work[bid & 7] += qt + 1;
        if (bh < 0 || bh >= per || qt < 0 || qt >= n) {
            printf("out of range: %s %ld %ld %ld: workgroup %ld -> head %d tile %d\n", what, a, b, c, (long)bid, bh, qt);
            return false;
        }
        if (seen[(size_t)bh * n + qt]++) {
            printf("twice: %s %ld %ld %ld: workgroup %ld -> head %d tile %d\n", what, a, b, c, (long)bid, bh, qt);
            return false;
        }
        ++hits;
    }
    if (hits != per * n) {
        printf("missed: %s %ld %ld %ld: %ld of %ld tiles\n", what, a, b, c, (long)hits, (long)(per * n));
        return false;
    }
    // Balance.  Over two consecutive rows of S list positions every slice
    // takes the same total weight, so slices of one group differ only by
    // their last, odd row: at most S tiles of a group's lightest rows, whose
    // weight is at most a few diagonal blocks each: bounded here by 2 * S * S
    // blocks per slice, U slices per XCD (dense groups are all full).  Whole-
    // group orders (S = 1, varlen) are balanced only on average and are not
    // held to it.
    if (d.S > 1) {
        const int64_t mx = *std::max_element(work, work + 8), mn = *std::min_element(work, work + 8);
        const int64_t bound = (int64_t)d.U * 2 * d.S * d.S;
        worst_gap = std::max(worst_gap, mx - mn);
        if (mx - mn > bound) {
            printf("unbalanced: %s %ld %ld %ld: XCD work %ld .. %ld (bound %ld)\n", what, a, b, c, (long)mn,
                   (long)mx, (long)bound);
            return false;
        }
    }
    return true;
}

static bool dense_causal(int B, int H, int N, bool four_wave) {
    const int64_t br = four_wave ? 128 : 256, slots = four_wave ? 64 : 32;
    const int64_t n = (N + br - 1) / br, per = (int64_t)B * H;
    int64_t G = std::min<int64_t>(per, (slots + n - 1) / n);
    Deal d{};
    int64_t grid = 0;
    ++n_shapes;
    if (!causal_deal(per, G, n, slots, d, grid) || grid > INT32_MAX) return true;   // plain order
    ++n_dealt;
    return covers(per, G, n, d, grid, four_wave ? "128-row tiles B H N" : "256-row tiles B H N", B, H, N);
}

// The backward's dK/dV grid: 128-key tiles, one workgroup per CU (32 slots
// per XCD), units of (batch, K/V head, part).  (Its dQ grid takes one of
// the two dense forms above.)
static bool dkdv_causal(int units, int N) {
    const int64_t n = (N + 127) / 128, slots = 32;
    int64_t G = std::min<int64_t>(units, (slots + n - 1) / n);
    Deal d{};
    int64_t grid = 0;
    ++n_shapes;
    if (!causal_deal(units, G, n, slots, d, grid) || grid > INT32_MAX) return true;
    ++n_dealt;
    return covers(units, G, n, d, grid, "dkdv units N", units, N, 0);
}

// Causal varlen batches of nearly equal lengths: the dense causal rule, in
// either tile form.
static bool varlen_equal_causal(int pairs, int max_seqlen, bool four_wave) {
    const int64_t br = four_wave ? 128 : 256, slots = four_wave ? 64 : 32;
    const int64_t n = (max_seqlen + br - 1) / br;
    int64_t G = std::min<int64_t>(pairs, (slots + n - 1) / n);
    Deal d{};
    int64_t grid = 0;
    ++n_shapes;
    if (!causal_deal(pairs, G, n, slots, d, grid) || grid > INT32_MAX) return true;
    ++n_dealt;
    return covers(pairs, G, n, d, grid, "varlen equal pairs max_seqlen", pairs, max_seqlen, four_wave);
}

static bool varlen(int n_seq, int H, int max_seqlen, bool four_wave) {
    const int64_t br = four_wave ? 128 : 256, slots = four_wave ? 64 : 32;
    const int64_t n = (max_seqlen + br - 1) / br, pairs = (int64_t)n_seq * H;
    const int64_t G = std::min<int64_t>(pairs, (slots + n - 1) / n);
    const int64_t ng = (pairs + G - 1) / G;
    int64_t grid = 0;
    const Deal d = ng < 32 ? make_deal(pairs, G, n, 8, true, grid) : make_deal(pairs, G, n, 1, false, grid);
    ++n_shapes;
    ++n_dealt;
    return covers(pairs, G, n, d, grid, four_wave ? "varlen 128-row n_seq H max_seqlen" : "varlen 256-row n_seq H max_seqlen",
                  n_seq, H, max_seqlen);
}

int main() {
    const int Ns[] = {1, 31, 100, 128, 129, 255, 256, 1000, 2048, 4095, 4096, 4097,
                      8192, 8193, 12345, 16384, 65536, 131073};
    for (int B = 1; B <= 9; ++B)
        for (int H = 1; H <= 40; ++H)
            for (int N : Ns)
                for (int f = 0; f < 2; ++f)
                    if (!dense_causal(B, H, N, f)) return 1;
    const int longest[] = {1 << 20, 3000001, (1 << 23) - 1};
    for (int H = 1; H <= 12; ++H)
        for (int N : longest)
            for (int f = 0; f < 2; ++f)
                if (!dense_causal(1, H, N, f)) return 1;
    for (int u = 1; u <= 72; ++u)
        for (int N : Ns)
            if (!dkdv_causal(u, N)) return 1;
    const int Ls[] = {1, 100, 128, 129, 1000, 4096, 8192, 8193, 32768, 100000};
    for (int s = 2; s <= 40; ++s)
        for (int H = 1; H <= 16; ++H)
            for (int L : Ls)
                for (int f = 0; f < 2; ++f)
                    if (!varlen(s, H, L, f)) return 1;
    for (int f = 0; f < 2; ++f)
        if (!varlen(2, 1, (1 << 23) - 1001, f) || !varlen(2, 2, (1 << 23) - 1001, f)) return 1;
    for (int pr = 1; pr <= 72; ++pr)
        for (int L : Ls)
            for (int f = 0; f < 2; ++f)
                if (!varlen_equal_causal(pr, L, f)) return 1;
    for (int f = 0; f < 2; ++f)
        if (!varlen_equal_causal(1, (1 << 23) - 1, f)) return 1;
    printf("ok: %ld launch shapes, %ld with a dealt grid, largest XCD work gap %ld blocks\n", n_shapes, n_dealt,
           (long)worst_gap);
    return 0;
}
