// kernels_transpose.hip -- tiled transpose out[c][r] = in[r][c] for 2- and 4-byte
// elements.
//
// "CUDA tile" (applications section) uses the transpose as the second case of tiling:
// reading rows and writing rows of the transposed matrix cannot both be coalesced
// directly, so a tile goes through shared memory, and a padded row keeps the
// column-wise accesses from colliding in one bank.  Here:
//   * a workgroup of 256 threads owns a 64 x 64 tile of `in` (16 KiB of fp32, 8 KiB of
//     16-bit elements) and loops over several tiles down a column of tiles;
//   * it reads the tile in 16-byte chunks along the rows of `in` (V = 16 / E elements a
//     chunk, 64 / V chunks a row), writes them to LDS as 16-byte chunks, and then each
//     thread gathers V consecutive rows of one column (one 16-byte chunk of a row of
//     `out`) with V single-element LDS reads, and stores it with one 16-byte store;
//   * instead of the page's one-element padding, chunk c of LDS row r sits at
//     c ^ ((r / V) % (64 / V)): the V-row groups a wave reads at one column then land in
//     distinct 16-byte slots of their rows, so a read instruction touches distinct banks
//     while the 16-byte writes stay whole (a padded row would break their alignment).
// Edges: chunks that are not wholly inside the matrix, or whose addresses are not
// 16-byte aligned (base pointer or leading dimension), go element by element with
// bounds checks; the rest of the tile keeps the vector path.
#include "device.h"

namespace mhg {
namespace transpose {

constexpr int T = 64;            // tile edge in elements
constexpr int NT = 256;          // threads a workgroup
constexpr int TILES_PER_WG = 4;  // tiles a workgroup walks down a column of tiles

template <int E>
struct Elem;
template <>
struct Elem<2> { typedef uint16_t type; };
template <>
struct Elem<4> { typedef uint32_t type; };

template <int E>
__global__ void __launch_bounds__(NT) transpose_tiles(const void *in_, void *out_, int64_t rows, int64_t cols,
                                                      int64_t ld_in, int64_t ld_out, int vec_in, int vec_out,
                                                      int64_t tiles_r, int64_t tiles_c) {
  typedef typename Elem<E>::type U;
  constexpr int V = 16 / E;            // elements a 16-byte chunk
  constexpr int CPR = T / V;           // chunks a tile row
  constexpr int CHUNKS = T * CPR;      // chunks a tile
  __shared__ __attribute__((aligned(16))) U tile[T * T];
  const U *in = static_cast<const U *>(in_);
  U *out = static_cast<U *>(out_);
  const int tid = threadIdx.x;
  // Workgroup -> (column of tiles, first tile row): the tile column varies fastest, so
  // consecutive workgroups read neighbouring pieces of the same rows.
  const int64_t tc = int64_t(blockIdx.x) % tiles_c;
  const int64_t tr0 = int64_t(blockIdx.x) / tiles_c * TILES_PER_WG;
  for (int t = 0; t < TILES_PER_WG; ++t) {
    const int64_t tr = tr0 + t;
    if (tr >= tiles_r) break;
    const int64_t r0 = tr * T, c0 = tc * T;
    if (t > 0) __syncthreads();   // the previous tile's reads of LDS are done
    // Read: chunk q = row (q / CPR), chunk (q % CPR) of the row.
#pragma unroll
    for (int k = 0; k < CHUNKS / NT; ++k) {
      const int q = tid + NT * k, r = q / CPR, c = q % CPR;
      const int64_t gr = r0 + r, gc = c0 + int64_t(V) * c;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (gr < rows) {
        if (vec_in && gc + V <= cols) {
          v = *reinterpret_cast<const u32x4 *>(in + gr * ld_in + gc);
        } else {
          U e[V];
#pragma unroll
          for (int i = 0; i < V; ++i) e[i] = gc + i < cols ? in[gr * ld_in + gc + i] : U(0);
          v = __builtin_bit_cast(u32x4, e);
        }
      }
      const int slot = c ^ ((r / V) % CPR);
      *reinterpret_cast<u32x4 *>(&tile[r * T + V * slot]) = v;
    }
    __syncthreads();
    // Write: output chunk q = output row j = q / CPR (input column c0 + j), chunk
    // (q % CPR) = input rows V (q % CPR) .. + V - 1.
#pragma unroll
    for (int k = 0; k < CHUNKS / NT; ++k) {
      const int q = tid + NT * k, j = q / CPR, rc = q % CPR;
      U e[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int r = V * rc + i;
        const int slot = (j / V) ^ ((r / V) % CPR);
        e[i] = tile[r * T + V * slot + j % V];
      }
      const int64_t orow = c0 + j, ocol = r0 + int64_t(V) * rc;
      if (orow >= cols) continue;
      if (vec_out && ocol + V <= rows) {
        *reinterpret_cast<u32x4 *>(out + orow * ld_out + ocol) = __builtin_bit_cast(u32x4, e);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (ocol + i < rows) out[orow * ld_out + ocol + i] = e[i];
      }
    }
  }
}

template __global__ void transpose_tiles<2>(const void *, void *, int64_t, int64_t, int64_t, int64_t, int, int,
                                            int64_t, int64_t);
template __global__ void transpose_tiles<4>(const void *, void *, int64_t, int64_t, int64_t, int64_t, int, int,
                                            int64_t, int64_t);

}  // namespace transpose

// out (cols x rows, leading dimension ld_out) = transpose of in (rows x cols, ld_in);
// the host has checked the arguments.
hipError_t launch_transpose(const void *in, void *out, int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                            int elem_bytes, hipStream_t s) {
  using namespace transpose;
  const int64_t tiles_r = (rows + T - 1) / T, tiles_c = (cols + T - 1) / T;
  const int64_t gy = (tiles_r + TILES_PER_WG - 1) / TILES_PER_WG;
  if (tiles_c * gy > 0x7fffffff) return hipErrorInvalidValue;
  const int V = 16 / elem_bytes;
  const bool vec_in = (reinterpret_cast<uintptr_t>(in) % 16 == 0) && (ld_in % V == 0);
  const bool vec_out = (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (ld_out % V == 0);
  const dim3 grid(static_cast<unsigned>(tiles_c * gy)), block(NT);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(transpose_tiles<4>, grid, block, 0, s, in, out, rows, cols, ld_in, ld_out, int(vec_in),
                       int(vec_out), tiles_r, tiles_c);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(transpose_tiles<2>, grid, block, 0, s, in, out, rows, cols, ld_in, ld_out, int(vec_in),
                       int(vec_out), tiles_r, tiles_c);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mhg
