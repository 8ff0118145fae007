// Host-side probe of the LDS layouts the gfx950 kernels read (attn_tiles.h,
// attn_direct.h): prints, for every tile type and operand read, the byte address
// each of the 64 lanes reads, one read instruction per line:
//   <layout> <read kind: row|tr> <bytes per lane> <64 addresses>
// tests/test_lds_layout.py checks them against the LDS bank model.
#include <stdio.h>

#include "../causal_attention_flash_amd/csrc/attn_direct.h"

using namespace attn;

template <class TILE, int D>
static void emit(const char* name) {
    // row operand reads: rows r0 + n, columns 16 ks + 8 h (16 bytes per lane)
    for (int r0 = 0; r0 < 64; r0 += 32)
        for (int ks = 0; ks < D / 16; ++ks) {
            printf("%s row 16", name);
            for (int l = 0; l < 64; ++l) printf(" %d", 2 * TILE::at(r0 + (l & 31), ks * 16 + 8 * (l >> 5)));
            printf("\n");
        }
    // transposing reads: the lds_tr_operand lane map (8 bytes per lane)
    for (int r0 = 0; r0 < 64; r0 += 16)
        for (int db = 0; db < HeadDim<D>::DB; ++db)
            for (int e = 0; e < 2; ++e) {
                printf("%s tr 8", name);
                for (int l = 0; l < 64; ++l) {
                    const int g = l >> 4, j = l & 15;
                    const int row = r0 + 4 * (g >> 1) + (j >> 2) + 8 * e;
                    const int col = db * 32 + 16 * (g & 1) + 4 * (j & 3);
                    printf(" %d", 2 * TILE::at(row, col));
                }
                printf("\n");
            }
}

// fp8 K rows (D bytes per row, D / 2 16-bit slots): two 16-byte row reads per
// 64-wide step, lane (n, h) reading bytes 32 h .. 32 h + 31 of row n
template <class TILE, int D>
static void emit_fp8(const char* name) {
    for (int st = 0; st < D / 64; ++st)
        for (int part = 0; part < 2; ++part) {
            printf("%s row 16", name);
            for (int l = 0; l < 64; ++l)
                printf(" %d", 2 * TILE::at(l & 31, st * 32 + 16 * (l >> 5) + 8 * part));
            printf("\n");
        }
}

int main() {
    emit<DTile<32, 64, 4>, 64>("swizzled_d64");
    emit<DTile<32, 80, 4>, 80>("swizzled_d80");
    emit<DTile<32, 96, 4>, 96>("swizzled_d96");
    emit<DTile<32, 128, 4>, 128>("swizzled_d128");
    emit<RowTile<64, 64, 512>, 64>("padded_d64");
    emit<RowTile<64, 80, 512>, 80>("padded_d80");
    emit<RowTile<64, 96, 512>, 96>("padded_d96");
    emit<RowTile<32, 128, 256>, 128>("padded_d128");
    emit_fp8<DTile<64, 32, 4>, 64>("fp8_d64");
    emit_fp8<DTile<32, 64, 4>, 128>("fp8_d128");
    return 0;
}
