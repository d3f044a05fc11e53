"""Readers for the Shapes tables stored next to this file (see their headers)."""
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def _read(name):
    rows = []
    header = None
    with open(os.path.join(_HERE, name)) as f:
        for line in f:
            line = line.rstrip("\n")
            if not line or line.startswith("#"):
                continue
            cells = line.split("\t")
            if header is None:
                header = cells
                continue
            row = {}
            for key, cell in zip(header, cells):
                try:
                    row[key] = int(cell)
                except ValueError:
                    try:
                        row[key] = float(cell)
                    except ValueError:
                        row[key] = cell
            rows.append(row)
    return rows


def prefill_rows():
    return _read("attention_forward_shapes.tsv")


def decode_rows():
    return _read("paged_attention_decode_shapes.tsv")


def chunk_rows():
    return _read("chunk_delta_rule_output_shapes.tsv")
