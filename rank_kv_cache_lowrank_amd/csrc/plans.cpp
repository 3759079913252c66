// Host-only plans shared by the C ABI (abi.cpp) and the kernel launchers: the shape of a rebase
// launch and the workspace sizes of the weighted SVD and the basis update. Kept out of the HIP
// sources so that a host-only build of the ABI layer (with the launchers stubbed) runs the same
// validation and sizing code.
#include "internal.h"

namespace lr {

// K steps of 32 old coordinates a rebase workgroup is instantiated for, and the W blocks of 16 new
// coordinates one multiplying wave holds in registers for each.
static int rb_nks_t(int r_old) {
  const int nks = (r_old + 31) / 32;
  return nks <= 4 ? 4 : (nks <= 8 ? 8 : (nks <= 12 ? 12 : 16));
}
static int rb_nb_max(int nks_t) { return nks_t == 16 ? 2 : (nks_t == 12 ? 3 : (nks_t == 8 ? 4 : 8)); }

void rebase_shape(int r_old, int r_new, RebaseShape* s) {
  s->nks_t = rb_nks_t(r_old);
  const int per = kRbConsumers * rb_nb_max(s->nks_t);   // blocks one workgroup holds
  const int nblk = (r_new + 15) / 16;
  const int nchunk = (nblk + per - 1) / per;
  const int blk_chunk = (nblk + nchunk - 1) / nchunk;
  s->nb = (blk_chunk + kRbConsumers - 1) / kRbConsumers;
  s->col_chunk = s->nb * kRbConsumers * 16;
  s->nchunk = (r_new + s->col_chunk - 1) / s->col_chunk;
  s->all = 0;
  // Where 4 consumer waves need several chunks (each re-reading the rows), 8 waves that also
  // load the ring, each with as many W blocks as its registers hold, need half as many (one
  // for ranks up to 384 at 12 K steps and up to 512 at 8).
  if (s->nchunk > 1 && s->nks_t >= 8) {
    const int nb = rb_nb_max(s->nks_t);
    const int cols = kRbAllWaves * nb * 16;
    const int nch = (r_new + cols - 1) / cols;
    if (nch < s->nchunk) {
      s->all = 1;
      s->nb = nb;
      s->col_chunk = cols;
      s->nchunk = nch;
    }
  }
}

int svd_nsplit(int n) {
  int s = (n + 255) / 256;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

size_t svd_workspace_bytes(int n, int D) {
  const size_t dd = (size_t)D * D * 4;
  return (size_t)svd_nsplit(n) * dd + 3 * dd + (size_t)(D / kJs) * kJs * kJs * 4 +
         (size_t)(D / kRqRows + 1) * D * 8 + (size_t)D * 4 + 1024;
}

size_t svd_workspace_stride(int n, int D) { return (svd_workspace_bytes(n, D) + 255) / 256 * 256; }

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Basis update workspace: staged rows, unit weights, the SVD's own workspace, B' (float32), the
// spectrum.
size_t basis_update_workspace_bytes(int r, int n, int D) {
  const int m = r + n;
  return align256((size_t)m * D * 2) + align256((size_t)m * 4) + align256(svd_workspace_bytes(m, D)) +
         align256((size_t)D * D * 4) + align256((size_t)D * 4);
}

}  // namespace lr
