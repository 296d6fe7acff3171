/*
 * transpose_oracle.c -- the CPU oracle for the shared-tile matrix transpose
 * and for the global-memory sector model.
 *
 * TEST INFRASTRUCTURE ONLY, like gemm_oracle.c: nothing in the product path
 * may include, link, load or call it.
 *
 * What it follows:
 *   - "03 CUDA Shared Memory: Tiling, Bank Conflicts, and Reduction",
 *     section "Bank Conflict": the transpose example, whose result is the
 *     plain transpose out[c][r] = in[r][c] (a shared tile only reorders the
 *     copy; no arithmetic happens).
 *   - same page, section "Global Memory와 Coalescing": memory is moved in
 *     fixed-size, size-aligned sectors; the cost of one access of a group of
 *     lanes is the number of distinct sectors its bytes touch.
 *
 * Pins (CPU tests): transposing twice is the identity, the library
 * transpose, brute force on tiny shapes, untouched padding, and the sector
 * counts the page prints (128, 160 and 1024 bytes for 32 lanes of 4-byte
 * floats: aligned, shifted by one float, and 32 bytes apart).
 */
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* out (cols x rows, leading dimension ld_out) = transpose of in (rows x
 * cols, leading dimension ld_in): out[c*ld_out + r] = in[r*ld_in + c].
 * Words of out outside the cols x rows window are not written. */
int oracle_transpose(int64_t rows, int64_t cols, const float *in, int64_t ld_in,
                     float *out, int64_t ld_out)
{
    if (rows < 0 || cols < 0)
        return ORACLE_BAD_ARG;
    if (ld_in < (cols > 1 ? cols : 1) || ld_out < (rows > 1 ? rows : 1))
        return ORACLE_BAD_ARG;
    if (rows > 0 && cols > 0 && (!in || !out))
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            out[c * ld_out + r] = in[r * ld_in + c];
    return ORACLE_OK;
}

/* Number of distinct sector_bytes-sized, sector_bytes-aligned sectors that
 * the accesses touch: lane l reads `width` bytes starting at byte address
 * addr[l].  Returns -1 on bad arguments. */
int64_t oracle_sectors_touched(int64_t lanes, const int64_t *addr, int64_t width,
                               int64_t sector_bytes)
{
    if (lanes < 0 || width < 1 || sector_bytes < 1 || (lanes > 0 && !addr))
        return -1;
    int64_t cap = lanes * ((width + sector_bytes - 1) / sector_bytes + 1);
    int64_t *seen = (int64_t *)malloc((size_t)(cap > 0 ? cap : 1) * sizeof *seen);
    if (!seen)
        return -1;
    int64_t n = 0;
    for (int64_t l = 0; l < lanes; ++l) {
        if (addr[l] < 0) {
            free(seen);
            return -1;
        }
        for (int64_t s = addr[l] / sector_bytes; s <= (addr[l] + width - 1) / sector_bytes; ++s) {
            int dup = 0;
            for (int64_t e = 0; e < n; ++e)
                if (seen[e] == s) { dup = 1; break; }
            if (!dup)
                seen[n++] = s;
        }
    }
    free(seen);
    return n;
}
