// Host-side rendering of one attention layer's visibility, for auditing the mask rules
// ("Attention mask layout" of the DeepSeek-V4 model page: the sliding, CSA and HCA mask
// diagrams of a 16-token example, and the audit script described under them, which draws the
// masks, prints a terminal grid and dumps the indexer's per-query selections).
//
// Rows are queries; columns are the window keys (sequence positions) followed by one column
// per compressed entry C_w, i.e. the entry-visibility view rather than the gather slots.
// Cell states: window key visible, entry selected by the indexer (CSA) or visible (HCA),
// entry visible but not selected (CSA), masked, and "selected but not visible" (an index list
// that breaks the causal rule: flagged, never expected).
#include <stdio.h>

#include <string>
#include <vector>

#include "launch.h"

namespace dsv4 {

namespace {

enum Cell : unsigned char { kMasked = 0, kWindow = 1, kSelected = 2, kVisibleOnly = 3, kBad = 4 };

struct Grid {
  int rows = 0, n_pos = 0, n_ent = 0;
  std::vector<unsigned char> cells;  // [rows][n_pos + n_ent]
  std::vector<std::vector<int>> lists;  // CSA: each query's list as given (HCA: visible entries)
  std::vector<long long> pos;           // sequence index of each query
  unsigned char at(int r, int c) const { return cells[static_cast<size_t>(r) * (n_pos + n_ent) + c]; }
};

long long visible_entries(long long p, int m, int n_entries) {
  const long long v = (p + 1) / m;
  return v < n_entries ? v : n_entries;
}

Grid build(const MaskDumpArgs& a) {
  Grid g;
  g.rows = a.S;
  g.n_pos = static_cast<int>(a.q_pos0 + a.S);
  g.n_ent = a.kind == 0 ? 0 : a.n_entries;
  const int width = g.n_pos + g.n_ent;
  g.cells.assign(static_cast<size_t>(g.rows) * width, kMasked);
  g.lists.resize(g.rows);
  g.pos.resize(g.rows);
  for (int t = 0; t < a.S; ++t) {
    const long long p = a.q_pos0 + t;
    g.pos[t] = p;
    unsigned char* row = &g.cells[static_cast<size_t>(t) * width];
    const long long lo = p - a.window + 1 > 0 ? p - a.window + 1 : 0;
    for (long long j = lo; j <= p; ++j) row[j] = kWindow;
    if (a.kind == 0) continue;
    const long long vis = visible_entries(p, a.m, a.n_entries);
    if (a.kind == 2) {  // HCA: every closed entry
      for (long long w = 0; w < vis; ++w) {
        row[g.n_pos + w] = kSelected;
        g.lists[t].push_back(static_cast<int>(w));
      }
      continue;
    }
    for (long long w = 0; w < vis; ++w) row[g.n_pos + w] = kVisibleOnly;  // CSA candidates
    const int* lst = a.topk_idx + static_cast<size_t>(t) * a.k;
    for (int i = 0; i < a.k; ++i) {
      const int e = lst[i];
      g.lists[t].push_back(e);
      if (e < 0) continue;  // -1 sentinel: an empty slot
      if (e < vis) row[g.n_pos + e] = kSelected;
      else if (e < g.n_ent) row[g.n_pos + e] = kBad;
    }
  }
  return g;
}

const char* kind_name(int kind) {
  return kind == 0 ? "sliding" : kind == 1 ? "CSA" : "HCA";
}

void header(std::string& out, const MaskDumpArgs& a) {
  char line[256];
  snprintf(line, sizeof(line), "%s layer: %d queries from position %lld, window %d", kind_name(a.kind), a.S,
           static_cast<long long>(a.q_pos0), a.window);
  out += line;
  if (a.kind != 0) {
    snprintf(line, sizeof(line), ", rate m=%d, %d entries%s", a.m, a.n_entries, a.kind == 1 ? "" : " (no indexer)");
    out += line;
    if (a.kind == 1) {
      snprintf(line, sizeof(line), ", top-%d", a.k);
      out += line;
    }
  }
  out += "\n";
}

std::string text(const MaskDumpArgs& a, const Grid& g, bool ansi) {
  std::string out;
  header(out, a);
  out += ansi ? "legend: \x1b[34m#\x1b[0m window key, \x1b[32m#\x1b[0m selected/visible entry, "
                "\x1b[33m:\x1b[0m visible, not selected, . masked, \x1b[31m!\x1b[0m selected but not visible\n"
              : "legend: # window key, @ selected/visible entry, : visible, not selected, . masked, "
                "! selected but not visible\n";
  for (int t = 0; t < g.rows; ++t) {
    char lab[32];
    snprintf(lab, sizeof(lab), "%6lld ", static_cast<long long>(g.pos[t]));
    out += lab;
    for (int c = 0; c < g.n_pos + g.n_ent; ++c) {
      if (c == g.n_pos && g.n_ent > 0) out += " |";
      const unsigned char v = g.at(t, c);
      if (!ansi) {
        out += v == kWindow ? '#' : v == kSelected ? '@' : v == kVisibleOnly ? ':' : v == kBad ? '!' : '.';
      } else {
        switch (v) {
          case kWindow: out += "\x1b[34m#\x1b[0m"; break;
          case kSelected: out += "\x1b[32m#\x1b[0m"; break;
          case kVisibleOnly: out += "\x1b[33m:\x1b[0m"; break;
          case kBad: out += "\x1b[31m!\x1b[0m"; break;
          default: out += '.';
        }
      }
    }
    out += "\n";
  }
  return out;
}

std::string svg(const MaskDumpArgs& a, const Grid& g) {
  const int cell = 12, gap = g.n_ent > 0 ? cell : 0, left = 56, top = 36;
  const int width = left + (g.n_pos + g.n_ent) * cell + gap + 8;
  const int height = top + g.rows * cell + 8;
  std::string out;
  char buf[320];
  snprintf(buf, sizeof(buf),
           "<svg xmlns=\"http://www.w3.org/2000/svg\" width=\"%d\" height=\"%d\" font-family=\"monospace\" "
           "font-size=\"10\">\n",
           width, height);
  out += buf;
  std::string title;
  header(title, a);
  title.pop_back();  // the newline
  snprintf(buf, sizeof(buf), "<text x=\"4\" y=\"14\">%s</text>\n", title.c_str());
  out += buf;
  snprintf(buf, sizeof(buf), "<text x=\"%d\" y=\"30\">keys</text>\n", left);
  out += buf;
  if (g.n_ent > 0) {
    snprintf(buf, sizeof(buf), "<text x=\"%d\" y=\"30\">entries C_w</text>\n", left + g.n_pos * cell + gap);
    out += buf;
  }
  for (int t = 0; t < g.rows; ++t) {
    const int y = top + t * cell;
    snprintf(buf, sizeof(buf), "<text x=\"4\" y=\"%d\">%lld</text>\n", y + cell - 2, static_cast<long long>(g.pos[t]));
    out += buf;
    for (int c = 0; c < g.n_pos + g.n_ent; ++c) {
      const unsigned char v = g.at(t, c);
      const char* fill = v == kWindow ? "#3b6fd4" : v == kSelected ? "#2e9e44" : v == kVisibleOnly ? "#f2d16b"
                                                                       : v == kBad ? "#d43b3b" : "#eeeeee";
      const int x = left + c * cell + (c >= g.n_pos ? gap : 0);
      snprintf(buf, sizeof(buf),
               "<rect x=\"%d\" y=\"%d\" width=\"%d\" height=\"%d\" fill=\"%s\" stroke=\"#ffffff\" "
               "data-q=\"%d\" data-c=\"%d\" data-state=\"%d\"/>\n",
               x, y, cell, cell, fill, t, c, static_cast<int>(v));
      out += buf;
    }
  }
  out += "</svg>\n";
  return out;
}

std::string lists(const MaskDumpArgs& a, const Grid& g) {
  std::string out;
  header(out, a);
  char buf[64];
  for (int t = 0; t < g.rows; ++t) {
    const long long p = g.pos[t];
    const long long vis = a.kind == 0 ? 0 : visible_entries(p, a.m, a.n_entries);
    snprintf(buf, sizeof(buf), "query %lld (visible entries %lld):", p, vis);
    out += buf;
    int sentinels = 0;
    for (int e : g.lists[t]) {
      snprintf(buf, sizeof(buf), " %d", e);
      out += buf;
      sentinels += e < 0;
    }
    if (a.kind == 1 && sentinels > 0) {
      snprintf(buf, sizeof(buf), "   [%d empty slot%s]", sentinels, sentinels == 1 ? "" : "s");
      out += buf;
    }
    out += "\n";
  }
  return out;
}

}  // namespace

std::string render_mask(const MaskDumpArgs& a) {
  const Grid g = build(a);
  switch (a.format) {
    case 0: return text(a, g, false);
    case 1: return text(a, g, true);
    case 2: return svg(a, g);
    default: return lists(a, g);
  }
}

}  // namespace dsv4
