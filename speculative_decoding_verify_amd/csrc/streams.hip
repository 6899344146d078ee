// Multi-codebook stream bookkeeping on top of the verify pass ("An Efficient vLLM-Based
// Inference Pipeline for Unified Audio Understanding and Generation", page 2: the delay
// pattern and its de-interleave, the primary / auxiliary decomposition, the phase state
// machine with its dynamic vocabulary mask and the drain sub-phase).
//
// phase_mask_kernel: per logit row, the partition of the unmasked argmax (the row's
// modality) and the argmax under the mask of the session's phase at the start of the
// pass, or -1 where the row leaves that phase (acceptance stops there).
// stream_commit_kernel: per session, the committed tokens of the pass (the accepted path
// plus the correction) in order through the phase machine; in the audio and drain
// phases each step's S codes go to the code matrix with stream s delayed by s steps.
#include "common.h"
#include "kernels.h"

namespace sdv {

// Argmax over ids [lo, hi) of one row (lowest index on ties): a per-thread scan and a
// block reduction in a fixed pattern.  lo >= hi gives -1.
SDV_DEV void block_argmax(const float* z, int lo, int hi, float* sv, int* si, float& v_out, int& i_out) {
  float bv = -INFINITY;
  int bi = -1;
  for (int i = lo + (int)threadIdx.x; i < hi; i += blockDim.x) {
    const float v = z[i];
    if (bi < 0 || v > bv) {   // ascending i per thread: ties keep the lower index
      bv = v;
      bi = i;
    }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const float v = sv[threadIdx.x + o];
      const int i = si[threadIdx.x + o];
      const int j = si[threadIdx.x];
      if (i >= 0 && (j < 0 || v > sv[threadIdx.x] || (v == sv[threadIdx.x] && i < j))) {
        sv[threadIdx.x] = v;
        si[threadIdx.x] = i;
      }
    }
    __syncthreads();
  }
  v_out = sv[0];
  i_out = si[0];
  __syncthreads();
}

// one workgroup per (logit row r, session b); row ids are id_offset .. id_offset + n_ids - 1
__global__ __launch_bounds__(256) void phase_mask_kernel(PhaseMaskArgs a) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int r = blockIdx.x, b = blockIdx.y;
  const float* z = a.logits + ((size_t)b * a.R + r) * a.row_stride;
  const StreamCfgDev& c = a.cfg;
  float v;
  int i;
  block_argmax(z, 0, a.n_ids, sv, si, v, i);
  const int id = i < 0 ? -1 : i + a.id_offset;
  const int mod = id < 0 ? STREAM_MOD_OTHER
                         : id < c.text_end ? STREAM_MOD_TEXT
                                           : (id >= c.base && id < c.base + c.Vc) ? STREAM_MOD_AUDIO : STREAM_MOD_OTHER;
  const int phase = a.phase[b], pos = a.phase_pos[b];
  const int k = a.depth[r];
  int out = -1;
  if (phase == STREAM_TEXT) {
    if (mod != STREAM_MOD_AUDIO) {
      int j;
      block_argmax(z, 0, min(c.text_end - a.id_offset, a.n_ids), sv, si, v, j);
      out = j < 0 ? -1 : j + a.id_offset;
    }
  } else if (phase == STREAM_TRANSITION) {
    out = pos + k < c.n_bridge ? c.bridge[pos + k] : -1;
  } else if (phase == STREAM_AUDIO) {
    const int lo = max(c.base - a.id_offset, 0), hi = min(c.base + c.Vc - a.id_offset, a.n_ids);
    int j;
    block_argmax(z, lo, hi, sv, si, v, j);
    out = j < 0 ? -1 : j + a.id_offset;
  } else {
    out = pos + k < c.S - 1 ? c.base + c.pad_code : -1;
  }
  if (threadIdx.x == 0) {
    a.argmax_out[(size_t)b * a.R + r] = out;
    if (a.modality_out) a.modality_out[(size_t)b * a.R + r] = mod;
  }
}

hipError_t launch_phase_mask(const PhaseMaskArgs& a, hipStream_t s) {
  phase_mask_kernel<<<dim3(a.R, a.B), 256, 0, s>>>(a);
  return hipGetLastError();
}

// Audio step t of session b: stream s carries frame t - s (kept below the segment's
// frame count once known, and below max_frames).
SDV_DEV void put_codes(const StreamCommitArgs& a, int b, int t, int frames, const int32_t* codes) {
  const StreamCfgDev& c = a.cfg;
  for (int s = 0; s < c.S; ++s) {
    const int f = t - s;
    if (f >= 0 && f < c.max_frames && (frames < 0 || f < frames))
      a.matrix[((size_t)b * c.S + s) * c.max_frames + f] = codes ? codes[s] : -1;
  }
}

// one thread per session: the committed steps are sequential by definition
__global__ __launch_bounds__(64) void stream_commit_kernel(StreamCommitArgs a) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= a.B) return;
  const StreamCfgDev& c = a.cfg;
  int phase = a.phase[b], pos = a.phase_pos[b], t = a.step[b], frames = a.frames[b];
  const int start_phase = phase;
  const int n = a.n[b], next = a.next[b];
  // logit index of a chunk row (rows that are not logit rows give -1)
  auto lidx = [&](int row) {
    for (int r = 0; r < a.R; ++r)
      if (a.logit_rows[r] == row) return r;
    return -1;
  };
  for (int i = 0; i <= n; ++i) {
    int tok;
    int pred_row = i == 0 ? a.L_a - 1 : a.path[(size_t)b * a.T + i - 1];
    if (i < n) tok = a.tokens[(size_t)b * a.T + a.path[(size_t)b * a.T + i]];
    else tok = next;
    if (tok < 0) break;
    const int li = lidx(pred_row);
    const int32_t* codes = (a.cb_argmax && li >= 0) ? a.cb_argmax + ((size_t)b * a.R + li) * c.S : nullptr;
    if (phase == STREAM_TEXT) {
    } else if (phase == STREAM_TRANSITION) {
      if (++pos == c.n_bridge) {
        phase = STREAM_AUDIO;
        pos = 0;
        t = 0;
        frames = -1;
      }
    } else if (phase == STREAM_AUDIO) {
      if (tok - c.base == c.eoa_code) {
        frames = t;
        put_codes(a, b, t, frames, codes);
        ++t;
        phase = STREAM_DRAIN;
        pos = 0;
      } else {
        put_codes(a, b, t, frames, codes);
        ++t;
      }
    } else {
      put_codes(a, b, t, frames, codes);
      ++t;
      if (++pos == c.S - 1) {
        phase = STREAM_TEXT;
        pos = 0;
      }
    }
  }
  // a text pass that stopped where the unmasked argmax was a codebook-0 id: switch
  if (next < 0 && start_phase == STREAM_TEXT && phase == STREAM_TEXT && a.modality) {
    const int stop_row = n == 0 ? a.L_a - 1 : a.path[(size_t)b * a.T + n - 1];
    const int li = lidx(stop_row);
    if (li >= 0 && a.modality[(size_t)b * a.R + li] == STREAM_MOD_AUDIO) {
      if (c.n_bridge > 0) {
        phase = STREAM_TRANSITION;
      } else {
        phase = STREAM_AUDIO;
        t = 0;
        frames = -1;
      }
      pos = 0;
    }
  }
  a.phase[b] = phase;
  a.phase_pos[b] = pos;
  a.step[b] = t;
  a.frames[b] = frames;
}

hipError_t launch_stream_commit(const StreamCommitArgs& a, hipStream_t s) {
  stream_commit_kernel<<<(a.B + 63) / 64, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sdv
