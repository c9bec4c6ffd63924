"""Generator variants for the ablation study.

"FusionRCG" (section V-B, Ablation Study) builds complete variant libraries from
one generator, toggling one component at a time: the axis-priority graph
construction, the DSA evaluation order, the stepwise spherical fusion, and the
adaptive choice between its register-only and buffered tiers.  This module holds
the switch the generator consults; the product library is built with
``Variant()`` (every component on), and ``ablation.py`` builds the others into
libraries of their own.

On this library's mapping the components are:
  topology    graph of the lane tier (one quartet per lane, whole recurrence graph
              in the lane).  "ket_first": a node with f != 0 is lowered on the ket
              side, then bra nodes down to [00|00] (the shipping graph);
              "alg1": the printed axis-priority rule of Algorithm 1, the highest
              axis on which either side is non-zero, ket side first at that axis;
              "bra_first": lower e first, then f (the conventional order, x before
              y before z).  The lane-group tiers give each lane one bra component,
              which fixes the ket-first shape there, so the graph variants are
              built with every class in the lane tier ("lane_*").
  schedule    "dsa": the liveness-aware list scheduler (section III-A, Eq. (7));
              "topo": a plain topological order of the same graph.
  sph_fusion  True: the spherical transform fused stepwise into the horizontal
              recurrences (section III-B, Eq. (14)); False: the Cartesian block is
              written out and transformed on all four indices afterwards (Eq. (17)).
  tiers       "adaptive": the library's routing; "lane": the one-quartet-per-lane
              tier for every class (the page's register-only Tier 1); "memory": the
              LDS-buffered memory tier for every class (its buffered Tier 2).
"""
from __future__ import annotations

from dataclasses import dataclass, asdict


@dataclass(frozen=True)
class Variant:
    name: str = "full"
    topology: str = "ket_first"
    schedule: str = "dsa"
    sph_fusion: bool = True
    tiers: str = "adaptive"

    def as_dict(self):
        return asdict(self)


VARIANTS = {
    "full": Variant(),
    "no_dsa": Variant(name="no_dsa", schedule="topo"),
    "no_sph_fusion": Variant(name="no_sph_fusion", sph_fusion=False),
    "memory_only": Variant(name="memory_only", tiers="memory"),
    "lane_only": Variant(name="lane_only", tiers="lane"),
    "lane_alg1": Variant(name="lane_alg1", tiers="lane", topology="alg1"),
    "lane_bra_first": Variant(name="lane_bra_first", tiers="lane", topology="bra_first"),
    "lane_no_dsa": Variant(name="lane_no_dsa", tiers="lane", schedule="topo"),
}

CURRENT = VARIANTS["full"]


def set_variant(v: Variant | str) -> Variant:
    """Make ``v`` the variant the generator emits; returns the previous one."""
    global CURRENT
    prev = CURRENT
    CURRENT = VARIANTS[v] if isinstance(v, str) else v
    return prev
