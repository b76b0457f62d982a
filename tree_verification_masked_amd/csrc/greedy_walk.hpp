// The greedy (T = 0) verification walk of one request, by one whole wavefront, shared
// by the sampler's greedy kernel and the row merge's launch (which runs it for the
// request whose rows it finished last).  Tree-verification notes
// (zhangshuibai.github.io), "Tree Verification 详解" part C: from the root, a drafted
// child is accepted when its token is the target's choice at its parent (the argmax
// at T = 0), siblings in ascending index; the walk ends at the first node with no
// accepted child, whose own choice is the bonus token (part G: at a leaf, the leaf's
// row).
#pragma once

#include "common.hpp"

namespace spectree {

struct GreedyArgs {
  const int32_t* parent;    // [batch, n_max]
  const int32_t* tokens;    // [batch, n_max]
  const int32_t* n_nodes;   // [batch]
  const float* row_max;     // [batch * n_max] target row maxima (NaN: an invalid row)
  const int32_t* row_argmax;
  int32_t n_max, vocab;
  int32_t* accepted_child;  // [batch, n_max]; null: no walk
  int32_t* term_token;
  int32_t *path_nodes, *out_tokens, *accept_len;  // all three or none
  int32_t* status;
};

// Lane i holds node slot i.  The accepted child of node cur is its first child, by
// index, whose token is cur's argmax: one ballot per step.  Writes accepted_child,
// term_token and (when given) the accepted path, as spec_accept_path derives it.
// agent: read the row statistics with agent-scope loads (written by other
// workgroups of the same launch).
template <bool kAgent>
__device__ inline void greedy_walk_wave(const GreedyArgs& g, int b) {
  const int lane = threadIdx.x & 63;
  const int64_t base = (int64_t)b * g.n_max;
  const int nb = g.n_nodes[b];
  const bool n_ok = nb >= 1 && nb <= g.n_max;
  const bool in = lane < g.n_max;
  const int par = in ? g.parent[base + lane] : -2;
  const int tok = in ? g.tokens[base + lane] : 0;
  int arg = -1;
  float mx = 0.0f;
  if (in) {
    if constexpr (kAgent) {
      arg = pub_load(&g.row_argmax[base + lane]);
      mx = pub_load(&g.row_max[base + lane]);
    } else {
      arg = g.row_argmax[base + lane];
      mx = g.row_max[base + lane];
    }
  }
  const bool live = n_ok && lane < nb;
  const bool bad_link = live && (lane == 0 ? par != -1 : (par < 0 || par >= lane));
  const bool bad_tok = live && lane > 0 && (tok < 0 || tok >= g.vocab);
  const unsigned long long m_link = __ballot(bad_link), m_tok = __ballot(bad_tok);
  int verdict = (!n_ok || m_link) ? SPEC_ERR_BAD_TREE : (m_tok ? SPEC_ERR_BAD_INPUT : 0);
  int oacc = SPEC_NODE_NOT_EVALUATED, oterm = SPEC_NODE_NOT_EVALUATED;
  int pn = lane == 0 ? 0 : -1, ot = -1;  // the path: slot len of path_nodes / out_tokens
  int cur = 0, len = 0;                  // the same in every lane
  for (int step = 0; verdict == 0 && step < nb; ++step) {
    const float m_cur = __shfl(mx, cur);
    const int am = __shfl(arg, cur);
    if (isnan(m_cur)) {
      verdict = SPEC_ERR_BAD_INPUT;
      break;
    }
    const unsigned long long kids = __ballot(lane > cur && lane < nb && par == cur && tok == am);
    const int acc = kids ? __ffsll(kids) - 1 : SPEC_NODE_NONE;
    if (lane == cur) oacc = acc;
    if (acc < 0) {
      if (lane == cur) oterm = am;
      if (lane == len) ot = am;
      break;
    }
    const int t_acc = __shfl(tok, acc);
    if (lane == len) ot = t_acc;
    ++len;
    if (lane == len) pn = acc;
    cur = acc;
  }
  if (verdict != 0) {
    oacc = lane == 0 ? SPEC_NODE_BAD_REQUEST : SPEC_NODE_NOT_EVALUATED;
    oterm = SPEC_NODE_NOT_EVALUATED;
    pn = ot = -1;
    len = -1;
    if (lane == 0) report(g.status, verdict);
  }
  if (in) {
    g.accepted_child[base + lane] = oacc;
    g.term_token[base + lane] = oterm;
    if (g.path_nodes) {
      g.path_nodes[base + lane] = pn;
      g.out_tokens[base + lane] = ot;
    }
  }
  if (lane == 0 && g.accept_len) g.accept_len[b] = len;
}

}  // namespace spectree
